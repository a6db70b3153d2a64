// FLARE forward kernels shared by both storage types, and the fp32 path.
//
//  combine           merges the split-N encode partials into Z (or Q' = Q + Z
//                    for FLARE++), in a fixed chunk order (deterministic).
//  encode_partial_f32, decode_f32
//                    fp32 storage and arithmetic throughout (no reduced-
//                    precision operands): one lane per latent in the encode,
//                    one lane per token in the decode, each with an exact
//                    online softmax (running maximum, rescaled sums).
//  copy_kernel       plain 16-byte-per-lane copy of known traffic.
//  fill_zero, widen, batch_sum
//                    elementwise helpers of the FLARE++ backward (a zero
//                    upstream gradient, dQ' widened to fp32, and the sum of
//                    its two stages' dQ in fp32, rounded once).
//
// Operator (FLARE skill page, steps 2 and 4; FLARE arXiv abstract):
// Z[m] = softmax_n(s <Q[m], K[n]>) V, Y[n] = softmax_m(s <Q[m], K[n]>) Z, with
// s = 1/sqrt(D); exponentials in base 2 on logits scaled by c = s log2(e).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "launch.h"

namespace flare {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Combine (FLARE++ residual included). One thread per (b, h, m) and four
// consecutive columns d (D is a multiple of 8):
//   mu* = max_c mu_c,  w_c = 2^(mu_c - mu*),
//   Z = sum_c w_c acc_c / sum_c w_c sig_c
// which is exactly the softmax over all N tokens (log-sum-exp merge), summed
// in chunk order (deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

template <int G>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int bh = blockIdx.y;
    const int D = a.D, D4 = D / 4;
    const int idx = blockIdx.x * 256 + threadIdx.x;  // (m, d/4)
    if (idx >= a.M * D4) return;
    const int m = idx / D4, d = 4 * (idx - m * D4);
    const int C = a.C, Mp = a.Mp;
    const int64_t row0 = (int64_t)bh * C * Mp + m;  // partial row of chunk 0; chunk c adds c*Mp
    const float* __restrict__ mu = a.in.mu + row0;
    const float* __restrict__ sg = a.in.sig + row0;
    const float* __restrict__ ac = a.in.acc + row0 * D + d;
    const int64_t sacc = (int64_t)Mp * D;
    // One pass over the chunks in groups of G: every load of a group is
    // issued before any use (one memory round trip per group), and a group
    // whose largest offset exceeds the running one rescales the sums first
    // (exact algebra: both are scaled by the same power of two).
    float mx = -INFINITY, den = 0.0f;
    f32x4c num = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < C; c0 += G) {
        float mv[G], sv[G];
        f32x4c av[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bool in = c0 + j < C;
            mv[j] = in ? mu[(int64_t)(c0 + j) * Mp] : -INFINITY;
            av[j] = in ? *(const f32x4c*)(ac + (int64_t)(c0 + j) * sacc) : f32x4c{0.0f, 0.0f, 0.0f, 0.0f};
            sv[j] = in ? sg[(int64_t)(c0 + j) * Mp] : 0.0f;
        }
        float gm = mx;
#pragma unroll
        for (int j = 0; j < G; ++j) gm = fmaxf(gm, mv[j]);
        if (gm > mx) {
            const float r = (mx == -INFINITY) ? 0.0f : exp2f(mx - gm);
            num *= r;
            den *= r;
            mx = gm;
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float w = (mv[j] == -INFINITY) ? 0.0f : exp2f(mv[j] - mx);
#pragma unroll
            for (int e = 0; e < 4; ++e) num[e] = fmaf(w, av[j][e], num[e]);
            den = fmaf(w, sv[j], den);
        }
    }
    f32x4c z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = num[e] / den;
    const int64_t o = (int64_t)bh * a.M * D + (int64_t)m * D + d;
    if (a.zmu && d == 0) a.zmu[(int64_t)bh * a.M + m] = mx;
    if (a.zsig && d == 0) a.zsig[(int64_t)bh * a.M + m] = den;
    if (a.mode == COMBINE_Z_F32 || (a.mode == COMBINE_Z_DTYPE && !a.bf16)) {
        *(f32x4c*)((float*)a.out + o) = z;
    } else if (a.mode == COMBINE_Z_DTYPE) {
        u16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = f32_to_bf16_rne(z[e]);
        *(u16x4*)((uint16_t*)a.out + o) = r;
    } else {
        const int h = bh % a.H;
        const int64_t qi = (int64_t)h * a.M * D + (int64_t)m * D + d;
        if (a.bf16) {
            const u16x4 qb = *(const u16x4*)((const uint16_t*)a.Q + qi);
            u16x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = f32_to_bf16_rne(__uint_as_float((uint32_t)qb[e] << 16) + z[e]);
            *(u16x4*)((uint16_t*)a.out + o) = r;
        } else {
            const f32x4c q = *(const f32x4c*)((const float*)a.Q + qi);
            *(f32x4c*)((float*)a.out + o) = q + z;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 encode partials: grid (C, BH, latent groups of blockDim.x); thread =
// latent. blockDim.x is M rounded up to 64, at most 256. K/V tiles of 64
// tokens go through LDS; each thread keeps its latent's exact running maximum,
// sum and accumulator.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void encode_partial_f32(EncodeArgs a) {
    constexpr int T = 64;
    __shared__ float kt[T * D], vt[T * D];
    const int tid = threadIdx.x, nth = blockDim.x;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int m = blockIdx.z * nth + tid;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M;
    const int n0 = chunk * a.chunk_len, n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    const float* Kb = (const float*)a.K + (int64_t)b * a.sb + (int64_t)h * a.sh;
    const float* Vb = (const float*)a.V + (int64_t)b * a.sb + (int64_t)h * a.sh;
    const float* Qb = (const float*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const bool active = m < M;
    float q[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = active ? Qb[(int64_t)m * D + d] : 0.0f;
        acc[d] = 0.0f;
    }
    float mu = -INFINITY, sig = 0.0f;
    for (int t0 = n0; t0 < n1; t0 += T) {
        const int nt = min(T, n1 - t0);
        for (int e = tid; e < nt * D; e += nth) {
            const int64_t g = (int64_t)(t0 + e / D) * a.sn + e % D;
            kt[e] = Kb[g];
            vt[e] = Vb[g];
        }
        __syncthreads();
        if (active) {
            for (int t = 0; t < nt; ++t) {
                float s = 0.0f;
#pragma unroll
                for (int d = 0; d < D; ++d) s = fmaf(q[d], kt[t * D + d], s);
                const float x = s * c;
                if (x > mu) {
                    const float alpha = (mu == -INFINITY) ? 0.0f : exp2f(mu - x);
                    sig *= alpha;
#pragma unroll
                    for (int d = 0; d < D; ++d) acc[d] *= alpha;
                    mu = x;
                }
                const float p = exp2f(x - mu);
                sig += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vt[t * D + d], acc[d]);
            }
        }
        __syncthreads();
    }
    if (active) {
        const int64_t r = ((int64_t)bh * gridDim.x + chunk) * a.Mp + m;
        a.out.mu[r] = mu;
        a.out.sig[r] = sig;
#pragma unroll
        for (int d = 0; d < D; ++d) a.out.acc[r * D + d] = acc[d];
    }
}

// ---------------------------------------------------------------------------
// fp32 decode: grid (token blocks of 256, BH); thread = token. Exact online
// softmax over the latents; Q and Z rows are read with wave-uniform addresses.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_f32(DecodeArgs a) {
    const int bh = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M;
    if (n >= N) return;
    const float c = a.c;
    const float* Qb = (const float*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const float* Zb = (const float*)a.Z + (int64_t)bh * M * D;
    const int64_t row = (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)n * a.sn;
    const float* kr = (const float*)a.K + row;
    float k[D], y[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        k[d] = kr[d];
        y[d] = 0.0f;
    }
    float nu = -INFINITY, tau = 0.0f;
    for (int m = 0; m < M; ++m) {
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(Qb[(int64_t)m * D + d], k[d], s);
        const float x = s * c;
        if (x > nu) {
            const float alpha = (nu == -INFINITY) ? 0.0f : exp2f(nu - x);
            tau *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) y[d] *= alpha;
            nu = x;
        }
        const float p = exp2f(x - nu);
        tau += p;
#pragma unroll
        for (int d = 0; d < D; ++d) y[d] = fmaf(p, Zb[(int64_t)m * D + d], y[d]);
    }
    float* yr = (float*)a.Y + row;
#pragma unroll
    for (int d = 0; d < D; ++d) yr[d] = y[d] / tau;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    size_t n16) {
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* __restrict__ dst, size_t n16) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) dst[i] = z;
}

template <typename T>
__device__ __forceinline__ float ld_f(const T* p) {
    if constexpr (sizeof(T) == 2) return __uint_as_float((uint32_t)(*(const uint16_t*)p) << 16);
    else return *(const float*)p;
}
template <typename T>
__device__ __forceinline__ void st_f(T* p, float v) {
    if constexpr (sizeof(T) == 2) *(uint16_t*)p = f32_to_bf16_rne(v);
    else *(float*)p = v;
}

// dst[i] = (float) src[i]
template <typename T>
__global__ __launch_bounds__(256) void widen_kernel(const T* __restrict__ src, float* __restrict__ dst, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = ld_f(src + i);
}

// dst[i] = base[i] + sum_b add[b * n + i], in fp32 over b in order, rounded once
template <typename T>
__global__ __launch_bounds__(256) void batch_sum_kernel(T* __restrict__ dst, const T* __restrict__ base,
                                                        const T* __restrict__ add, int B, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float v = ld_f(base + i);
        for (int b = 0; b < B; ++b) v += ld_f(add + (int64_t)b * n + i);
        st_f(dst + i, v);
    }
}

unsigned elementwise_blocks(int64_t n) { return (unsigned)std::min<int64_t>(8192, std::max<int64_t>(1, (n + 255) / 256)); }

template <int D>
hipError_t enc_f32(const EncodeArgs& a, hipStream_t s) {
    const int nth = enc_threads_f32(a.M);
    dim3 grid(a.C, a.BH, (a.M + nth - 1) / nth), block(nth);
    hipLaunchKernelGGL((encode_partial_f32<D>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t dec_f32(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((a.N + 255) / 256, a.BH), block(256);
    hipLaunchKernelGGL((decode_f32<D>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

// fp32 kernels are instantiated for head widths that are multiples of 8.
#define FLARE_F32_DISPATCH(FN, a, s)     \
    switch ((a).D) {                     \
        case 8: return FN<8>(a, s);      \
        case 16: return FN<16>(a, s);    \
        case 24: return FN<24>(a, s);    \
        case 32: return FN<32>(a, s);    \
        case 48: return FN<48>(a, s);    \
        case 64: return FN<64>(a, s);    \
        case 96: return FN<96>(a, s);    \
        case 128: return FN<128>(a, s);  \
        default: return hipErrorInvalidValue; \
    }

int enc_threads_f32(int M) { return M >= 256 ? 256 : (M + 63) / 64 * 64; }

hipError_t launch_encode_f32(const EncodeArgs& a, hipStream_t s) { FLARE_F32_DISPATCH(enc_f32, a, s) }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) { FLARE_F32_DISPATCH(dec_f32, a, s) }

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.D % 4 != 0) return hipErrorInvalidValue;
    dim3 grid((a.M * (a.D / 4) + 255) / 256, a.BH), block(256);
    // groups of 8 chunks when that covers them all (fewer registers), else 16
    if (a.C <= 8)
        hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s) {
    if (bytes % 16 != 0) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(elementwise_blocks((int64_t)n16)), dim3(256), 0, s, (u32x4*)dst, n16);
    return hipGetLastError();
}

hipError_t launch_widen(const void* src, float* dst, int64_t n, bool bf16, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(widen_kernel<uint16_t>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (const uint16_t*)src, dst, n);
    else
        hipLaunchKernelGGL(widen_kernel<float>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (const float*)src, dst, n);
    return hipGetLastError();
}

hipError_t launch_batch_sum(void* dst, const void* base, const void* add, int B, int64_t n, bool bf16, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(batch_sum_kernel<uint16_t>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (uint16_t*)dst,
                           (const uint16_t*)base, (const uint16_t*)add, B, n);
    else
        hipLaunchKernelGGL(batch_sum_kernel<float>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (float*)dst,
                           (const float*)base, (const float*)add, B, n);
    return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, n16);
    return hipGetLastError();
}

}  // namespace flare
