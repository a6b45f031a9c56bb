// append.hip -- write new token rows into the per-layer caches.
//
// MSA ("Add MiniMax-M3 (MSA: MiniMax Sparse Attention) support",
// Implementation): the index keys live in their own per-layer F32 cache next
// to the bf16 K/V cache; the append is an exact copy of the rows (or, for an
// fp16 index cache, one round-to-nearest-even conversion of each key).
// DSA ("deepseek2 : GLM-DSA sparse attention (lightning indexer)", What this
// does): indexer keys are Hadamard-rotated before they enter the F16 cache.
// The rotation here is the Sylvester-ordered fast Walsh-Hadamard transform
// carried out in fp64, where every partial sum of fp16 inputs is exact (they
// are multiples of 2^-24 below 2^23), scaled by 1/sqrt(128) in fp64 and
// rounded once to fp16 with round-to-nearest-even.
#include "common.hpp"

namespace msa {
namespace {

// fp64 -> fp16 bits, round to nearest, ties to even, from the IEEE binary64
// fields: the 53-bit significand is shifted down to the fp16 significand
// width (11 bits for normals, fewer for subnormals) with an RNE decision on
// the bits shifted out.
__device__ uint16_t f64_to_f16_bits_rne(double x) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
    const int e64 = static_cast<int>((u >> 52) & 0x7ff);
    const uint64_t frac = u & ((1ull << 52) - 1);
    if (e64 == 0x7ff) return sign | (frac ? 0x7e00 : 0x7c00);
    if (e64 == 0) return sign;                        // fp64 subnormals round to 0 in fp16
    const uint64_t sig = frac | (1ull << 52);         // value = sig * 2^(e64 - 1075)
    int e16 = e64 - 1023 + 15;                        // biased fp16 exponent if normal
    int shift = 42;                                   // 53-bit -> 11-bit significand
    if (e16 < 1) shift += 1 - e16;                    // subnormal: fewer bits kept
    if (shift > 63) return sign;
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (e16 < 1) return sign | static_cast<uint16_t>(q);   // q == 1024 encodes the min normal
    if (q == 2048) { q = 1024; ++e16; }
    if (e16 >= 31) return sign | 0x7c00;
    return sign | static_cast<uint16_t>((e16 << 10) | (q - 1024));
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
    return static_cast<double>(__builtin_bit_cast(_Float16, h));   // exact
}

// One workgroup of 128 threads per new row.
__global__ __launch_bounds__(128) void append_kernel(
    float* __restrict__ idx_k, uint16_t* __restrict__ idx_k16, uint16_t* __restrict__ dsa_k, uint16_t* __restrict__ k,
    uint16_t* __restrict__ v, Pager pg, const int32_t* __restrict__ stream,
    const int32_t* __restrict__ pos, const float* __restrict__ idx_k_new,
    const uint16_t* __restrict__ dsa_key_new, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, double inv_sqrt_n) {
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t slot = pg.row(stream[i], pos[i]);

    if (idx_k_new) {   // 4 x 128 f32 = 128 x 16 B
        const u32x4* src = reinterpret_cast<const u32x4*>(idx_k_new + i * kGroups * kIdxDim);
        if (idx_k16) {     // fp16 cache: 4 keys -> 8 B per thread
            const f32x4 x = __builtin_bit_cast(f32x4, src[tid]);
            typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
            const f16x4 h = __builtin_convertvector(x, f16x4);    // round to nearest even
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            reinterpret_cast<u32x2_t*>(idx_k16 + slot * kGroups * kIdxDim)[tid] = __builtin_bit_cast(u32x2_t, h);
        } else {
            reinterpret_cast<u32x4*>(idx_k + slot * kGroups * kIdxDim)[tid] = src[tid];
        }
    }
    if (tid < 64) {    // 4 x 128 bf16 = 64 x 16 B each
        if (k_new) {
            const u32x4* src = reinterpret_cast<const u32x4*>(k_new + i * kGroups * kHeadDim);
            reinterpret_cast<u32x4*>(k + slot * kGroups * kHeadDim)[tid] = src[tid];
        }
        if (v_new) {
            const u32x4* src = reinterpret_cast<const u32x4*>(v_new + i * kGroups * kHeadDim);
            reinterpret_cast<u32x4*>(v + slot * kGroups * kHeadDim)[tid] = src[tid];
        }
    }
    if (dsa_key_new && tid < 64) {
        // lane l holds elements l and l + 64 of the 128-point transform
        const uint16_t* x = dsa_key_new + i * kIdxDim;
        double e0 = f16_bits_to_f64(x[tid]);
        double e1 = f16_bits_to_f64(x[tid + 64]);
        double t = e0 + e1;                           // butterfly of span 64 (in lane)
        e1 = e0 - e1;
        e0 = t;
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {           // spans 32 .. 1 across lanes
            const double p0 = __shfl_xor(e0, h, 64);
            const double p1 = __shfl_xor(e1, h, 64);
            const bool upper = (tid & h) != 0;
            e0 = upper ? p0 - e0 : e0 + p0;
            e1 = upper ? p1 - e1 : e1 + p1;
        }
        uint16_t* dst = dsa_k + slot * kIdxDim;
        dst[tid] = f64_to_f16_bits_rne(e0 * inv_sqrt_n);
        dst[tid + 64] = f64_to_f16_bits_rne(e1 * inv_sqrt_n);
    }
}

}  // namespace

hipError_t launch_append(float* idx_k, uint16_t* idx_k16, uint16_t* dsa_k, uint16_t* k, uint16_t* v, const Pager& pg,
                         const int32_t* stream, const int32_t* pos, int64_t n_new,
                         const float* idx_k_new, const uint16_t* dsa_key_new,
                         const uint16_t* k_new, const uint16_t* v_new, hipStream_t s) {
    // The scale is computed on the host, as 1 / sqrt(128) in IEEE double.
    const double inv_sqrt_n = 1.0 / __builtin_sqrt(static_cast<double>(kIdxDim));
    hipLaunchKernelGGL(append_kernel, dim3(static_cast<unsigned>(n_new)), dim3(128), 0, s, idx_k,
                       idx_k16, dsa_k, k, v, pg, stream, pos, idx_k_new, dsa_key_new, k_new, v_new,
                       inv_sqrt_n);
    return hipGetLastError();
}

}  // namespace msa
