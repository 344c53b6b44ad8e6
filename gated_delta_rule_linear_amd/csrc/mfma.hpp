// Matrix-core helpers for gfx950: v_mfma_f32_16x16x32_bf16 fragments read from LDS.
//
// Lane layout of the 16x16x32 bf16 MFMA (64 lanes, g = lane / 16, j = lane % 16):
//   A (16 x 32): lane holds row j, k = 8g .. 8g+7
//   B (32 x 16): lane holds col j, k = 8g .. 8g+7
//   D (16 x 16): lane holds col j, rows 4g .. 4g+3 (f32x4)
// A fragment whose K index runs along the rows of a row-major LDS tile (for example
// the token index of a [token][feature] tile) is fetched with the LDS transpose read
// ds_read_b64_tr_b16: within each 16-lane group, lane L addresses row L/4, columns
// 4*(L%4) .. +3 of a 4-row block, and lane j receives column j of those 4 rows.
#pragma once

#include "common.hpp"

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Fragment from a row-major bf16 tile whose rows are the M (or N) index and whose
// columns are K: rows r0 .. r0+15, K = k0 .. k0+31. Needs pitch % 8 == 0.
__device__ __forceinline__ bf16x8_t frag_kc(const uint16_t* t, int pitch, int r0, int k0,
                                            int lane) {
    return *reinterpret_cast<const bf16x8_t*>(t + (r0 + (lane & 15)) * pitch + k0 +
                                              (lane >> 4) * 8);
}

// Fragment from a row-major bf16 tile whose rows are K and whose columns are the M (or
// N) index (transpose read): M/N = n0 .. n0+15, K = k0 .. k0+31. Needs pitch % 4 == 0.
__device__ __forceinline__ bf16x8_t frag_kr(const uint16_t* t, int pitch, int k0, int n0,
                                            int lane) {
    const int g = lane >> 4, L = lane & 15;
    const uint16_t* p = t + (k0 + g * 8 + (L >> 2)) * pitch + n0 + (L & 3) * 4;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * pitch));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}


// Store a D tile (rows m0.., cols n0..) transposed into a bf16 tile t[col][row]
// (8-byte write per lane: t[n0 + j][m0 + 4g .. +3]). Needs pitch % 4 == 0.
__device__ __forceinline__ void store_dT(uint16_t* t, int pitch, int m0, int n0, f32x4_t d,
                                         int lane) {
    uint2 w;
    w.x = pack_bf16x2(d[0], d[1]);
    w.y = pack_bf16x2(d[2], d[3]);
    *reinterpret_cast<uint2*>(t + (n0 + (lane & 15)) * pitch + m0 + (lane >> 4) * 4) = w;
}

// Load 8 consecutive bf16 (16 bytes) from global memory as raw bits.
__device__ __forceinline__ uint4 ld_g16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void unpack8(uint4 w, float (&f)[8]) {
    f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
    f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
    f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    uint4 w;
    w.x = pack_bf16x2(f[0], f[1]);
    w.y = pack_bf16x2(f[2], f[3]);
    w.z = pack_bf16x2(f[4], f[5]);
    w.w = pack_bf16x2(f[6], f[7]);
    return w;
}

// Value columns of a 16 NVT-column slice as seen by its NVT column tiles: tile ct,
// tile-local index j (0..15) -> column 4 NVT (j / 4) + 4 ct + j % 4. The lane group g
// of a D tile (rows 4 g .. 4 g + 3) then owns the 4 NVT contiguous columns 4 NVT g ..
// across all tiles, so value loads and output stores are 8 NVT-byte accesses. Also
// colmap(ct, 4 q + e) = colmap(ct, 4 q) + e. NVT = 1 is the identity.
template <int NVT>
__device__ __forceinline__ int colmap(int ct, int j) {
    return 4 * NVT * (j >> 2) + 4 * ct + (j & 3);
}
// Fragment from a row-major [K rows][columns] bf16 tile whose M/N index is tile ct's
// columns (LDS transpose read; each lane quad addresses 4 consecutive columns).
template <int NVT>
__device__ __forceinline__ bf16x8_t frag_kr_cols(const uint16_t* t, int pitch, int k0, int cb,
                                                 int ct, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const uint16_t* p = t + (k0 + g * 8 + (L >> 2)) * pitch + cb + colmap<NVT>(ct, 4 * (L & 3));
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * pitch));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}
// As frag_kr_cols for K = 32 kk .. 32 kk + 31, with the K slots in the order in which
// the matrix cores return a pair of 16 x 16 tiles of a 32-wide K range: slots 0..3 are
// K = 32 kk + 4 g + 0..3, slots 4..7 are K = 32 kk + 16 + 4 g + 0..3. Paired with a
// fragment packed straight from two D tiles (D rows = that K range), no transpose of
// the tiles is needed.
template <int NVT>
__device__ __forceinline__ bf16x8_t frag_kr_cols_pk(const uint16_t* t, int pitch, int kk, int cb,
                                                    int ct, int lane) {
    const int g = lane >> 4, L = lane & 15;
    const uint16_t* p = t + (32 * kk + 4 * g + (L >> 2)) * pitch + cb + colmap<NVT>(ct, 4 * (L & 3));
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 16 * pitch));
    const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}
// B fragment packed from two D tiles d0 (K = 32 kk + 4 g ..) and d1 (K = 32 kk + 16 + 4 g ..)
// in the slot order of frag_kr_cols_pk.
__device__ __forceinline__ bf16x8_t pack_pk(f32x4_t d0, f32x4_t d1) {
    const uint4 w = make_uint4(pack_bf16x2(d0[0], d0[1]), pack_bf16x2(d0[2], d0[3]),
                               pack_bf16x2(d1[0], d1[1]), pack_bf16x2(d1[2], d1[3]));
    return __builtin_bit_cast(bf16x8_t, w);
}

// Fragment from a row-major [columns][K] bf16 tile (S^T) whose M index is tile ct's
// columns.
template <int NVT>
__device__ __forceinline__ bf16x8_t frag_st(const uint16_t* t, int pitch, int cb, int ct, int k0,
                                            int lane) {
    return *reinterpret_cast<const bf16x8_t*>(t + (cb + colmap<NVT>(ct, lane & 15)) * pitch + k0 +
                                              (lane >> 4) * 8);
}
// D tile [M = tile ct's columns][N = rows n0 ..] to a row-major [rows][columns] tile.
template <int NVT>
__device__ __forceinline__ void store_rows(uint16_t* t, int pitch, int cb, int ct, int n0,
                                           f32x4_t d, int lane) {
    uint2 w;
    w.x = pack_bf16x2(d[0], d[1]);
    w.y = pack_bf16x2(d[2], d[3]);
    *reinterpret_cast<uint2*>(t + (n0 + (lane & 15)) * pitch + cb +
                              colmap<NVT>(ct, 4 * (lane >> 4))) = w;
}
// D tile [M = key rows i0 ..][N = tile ct's columns] to the [columns][keys] tile S^T.
template <int NVT>
__device__ __forceinline__ void store_st(uint16_t* t, int pitch, int i0, int cb, int ct,
                                         f32x4_t d, int lane) {
    uint2 w;
    w.x = pack_bf16x2(d[0], d[1]);
    w.y = pack_bf16x2(d[2], d[3]);
    *reinterpret_cast<uint2*>(t + (cb + colmap<NVT>(ct, lane & 15)) * pitch + i0 +
                              4 * (lane >> 4)) = w;
}

// Raw bits of one gate element (bf16 or fp32 storage), converted later so that a
// prefetch load is not consumed right after it is issued.
template <bool GB>
__device__ __forceinline__ uint32_t ld_gate_raw(const void* p, size_t i) {
    if constexpr (GB) return static_cast<const uint16_t*>(p)[i];
    else return static_cast<const uint32_t*>(p)[i];
}
template <bool GB>
__device__ __forceinline__ float gate_val(uint32_t raw) {
    return GB ? __uint_as_float(raw << 16) : __uint_as_float(raw);
}
// Eight consecutive gate elements, raw: GB -> w[0] holds 8 bf16; fp32 -> w[0], w[1].
template <bool GB>
__device__ __forceinline__ void ld_gate8_raw(const void* p, size_t i, uint4 (&w)[2]) {
    if constexpr (GB) {
        w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
        w[1] = make_uint4(0, 0, 0, 0);
    } else {
        w[0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i);
        w[1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i + 4);
    }
}
template <bool GB>
__device__ __forceinline__ void gate8_val(const uint4 (&w)[2], float (&f)[8]) {
    if constexpr (GB) {
        unpack8(w[0], f);
    } else {
        f[0] = __uint_as_float(w[0].x); f[1] = __uint_as_float(w[0].y);
        f[2] = __uint_as_float(w[0].z); f[3] = __uint_as_float(w[0].w);
        f[4] = __uint_as_float(w[1].x); f[5] = __uint_as_float(w[1].y);
        f[6] = __uint_as_float(w[1].z); f[7] = __uint_as_float(w[1].w);
    }
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0, 0, 0, 0); }

// Raw buffer access (stride 0) through a resource over [base, base + bytes): the
// memory unit returns zero for loads at offsets >= bytes and drops such stores, so
// ragged tails need no branches and every load and store is issued unconditionally
// (which keeps the compiler's memory-counter waits exact across the chunk loop).
// Offsets are byte offsets below 2^31.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
// 16-byte loads carry the sc0 cache-policy bit (workgroup-scope coherence); for
// chunk operands that several workgroups re-read from L2 it measured no slower, and
// up to 6% faster, than the default policy.
__device__ __forceinline__ uint4 buf_ld16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 1));
}
__device__ __forceinline__ uint2 buf_ld8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_ld4(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_ld2(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void buf_st2(rsrc_t r, uint32_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_st8(rsrc_t r, uint32_t off, uint2 v) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_st16(rsrc_t r, uint32_t off, uint4 v) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 0);
}
// Output stores (written once, never read back by the kernel): non-temporal, so the
// lines stream out instead of displacing the inputs the walk still reads from L2.
__device__ __forceinline__ void buf_st16_out(rsrc_t r, uint32_t off, uint4 v) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 2);
}
// The same with a constant byte offset folded into the instruction (0 .. 4095), for
// loops whose per-lane offset register stays fixed while the resource moves.
__device__ __forceinline__ uint4 buf_ld16_off(rsrc_t r, uint32_t off, int imm) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + uint32_t(imm), 0, 1));
}
__device__ __forceinline__ void buf_st8_off(rsrc_t r, uint32_t off, int imm, uint2 v) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, off + uint32_t(imm), 0, 0);
}
template <bool GB>
__device__ __forceinline__ uint32_t buf_ld_gate_off(rsrc_t r, uint32_t off) {
    if constexpr (GB) return buf_ld2(r, off);
    else return buf_ld4(r, off);
}
// One gate element (bf16 or fp32 storage) as raw bits, converted with gate_val.
template <bool GB>
__device__ __forceinline__ uint32_t buf_ld_gate(rsrc_t r, uint32_t index) {
    if constexpr (GB) return buf_ld2(r, index * 2u);
    else return buf_ld4(r, index * 4u);
}

// Workgroup id -> (sequence, tile) with the tiles of one sequence on one XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each with its own
// L2, so tiles that re-read the same q/k rows are placed at ids = xcd + 8 * slot.
struct XcdMap {
    int seq, tile;
    bool valid;
};
__device__ __forceinline__ XcdMap xcd_map(int bid, int ntiles, int nseq) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int tile = slot % ntiles, group = slot / ntiles;
    XcdMap m;
    m.seq = group * 8 + xcd;
    m.tile = tile;
    m.valid = m.seq < nseq;
    return m;
}
__host__ __device__ constexpr int xcd_grid(int ntiles, int nseq) {
    return ((nseq + 7) / 8) * 8 * ntiles;
}

}  // namespace la
