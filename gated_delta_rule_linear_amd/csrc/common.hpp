// Device helpers shared by the kernel translation units: storage-dtype loads and
// stores, and small wavefront utilities. gfx950 only (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace la {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming accesses that bypass cache retention (state read-modify-write)
__device__ __forceinline__ float4 load_nt4(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt4(float* p, float4 x) {
    f32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(uint32_t(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (low half = a), round to nearest even, in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// fp32 -> bf16 bit pattern, round to nearest even
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return uint16_t(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads, so loads issued ahead for
// the next chunk stay in flight across it. The memory clobber keeps the compiler
// from moving shared-memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Within one wave: make this wave's LDS writes visible to its own later LDS reads
// (a wave's LDS operations execute in order once issued).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Element i of an array stored as fp32 (bf16 == false) or bf16 bits.
__device__ __forceinline__ float load_elem(const void* p, size_t i, bool bf16) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i])
                : static_cast<const float*>(p)[i];
}

// Element i of an array whose storage type is fixed at compile time (float or bf16 bits):
// loaders that pick the type once per call keep their loads in one straight run.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
template <class T>
__device__ __forceinline__ float ld(const void* p, size_t i) {
    return to_f32(static_cast<const T*>(p)[i]);
}

__device__ __forceinline__ void store_elem(void* p, size_t i, float x, bool bf16) {
    if (bf16)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
    else
        static_cast<float*>(p)[i] = x;
}

// Four consecutive elements starting at i (i a multiple of 4; 8- or 16-byte access).
__device__ __forceinline__ float4 load4(const void* p, size_t i, bool bf16) {
    if (bf16) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    }
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}

__device__ __forceinline__ void store4(void* p, size_t i, float4 x, bool bf16) {
    if (bf16) {
        uint2 w;
        w.x = pack_bf16x2(x.x, x.y);
        w.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = x;
    }
}

// ELU(x) + 1 (alpha = 1): x + 1 for x > 0, exp(x) otherwise. The feature map of
// normalized linear attention; it keeps features positive.
__device__ __forceinline__ float elu_plus_one(float x) { return x > 0.f ? x + 1.f : expf(x); }

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar) value so
// that control flow depending on it compiles to scalar branches.
// Tokens of sequence seq = s H + h. A dense [B, H, N, d] layout holds them at seq N,
// N of them. A packed variable-length batch (one [1, H, N, d] layout, cu the nseq + 1
// cumulative sequence lengths) holds sequence s of head h at h N + cu[s], cu[s + 1] -
// cu[s] of them: the state restarts at every boundary. Offsets are clamped to the
// head's N tokens and lengths to maxlen, so no access leaves the buffers whatever cu
// holds.
struct SeqSpan {
    size_t base;
    int len;
};
typedef const __attribute__((address_space(4))) int32_t const_i32_t;
__device__ __forceinline__ SeqSpan seq_span(int seq, int H, int N, int maxlen, const int32_t* cu) {
    if (cu == nullptr) return SeqSpan{size_t(seq) * size_t(N), N};
    const int s = seq / H, h = seq - s * H;
    // the bounds are read-only for the whole call: read them through the constant address
    // space (scalar loads), so that they are not counted with the vector memory loads
    const_i32_t* c = (const_i32_t*)(cu);
    const int st = min(max(c[s], 0), N);
    const int en = min(max(c[s + 1], st), N);
    return SeqSpan{size_t(h) * size_t(N) + size_t(st), min(en - st, maxlen)};
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Natural log and exp on the hardware transcendental units (log2 / exp2), a few ulp.
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * 0.69314718f; }
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504f); }

// ELU(x) + 1 with the hardware exponential (a few ulp; used where operands are rounded
// to bf16), branch-free: max(x, 0) + exp(min(x, 0)), which is x + 1 for x > 0 (the
// exponential of 0 is exactly 1) and exp(x) otherwise.
__device__ __forceinline__ float elu_plus_one_fast(float x) {
    return fmaxf(x, 0.f) + fast_exp(fminf(x, 0.f));
}

// DPP lane permutation of a float: lanes outside the enabled rows/banks (or with no
// source lane) receive 0.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, false));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane shifts: shifts of
// 1, 2, 4, 8 within each row of 16 lanes, then row 15 / lane 31 broadcasts across rows.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += dpp_f<0x111, 0xf, 0xf>(x);  // row_shr:1
    x += dpp_f<0x112, 0xf, 0xf>(x);  // row_shr:2
    x += dpp_f<0x114, 0xf, 0xf>(x);  // row_shr:4
    x += dpp_f<0x118, 0xf, 0xf>(x);  // row_shr:8
    x += dpp_f<0x142, 0xa, 0xf>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_f<0x143, 0xc, 0xf>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

}  // namespace la
