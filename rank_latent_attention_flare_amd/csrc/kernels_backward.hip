// Backward of the FLARE forward (gradients of Q, K and V), fp32 arithmetic on
// fp32 or bf16 storage.
//
// With l[m][n] = s <Q[m], K[n]> (s = 1/sqrt(D)), the encode softmax
// A[m][n] = softmax_n(l[m][.]), Z = A V, the decode softmax
// Bt[n][m] = softmax_m(l[.][n]) and Y = Bt Z (FLARE skill page, steps 2 and 4;
// FLARE arXiv abstract), the chain rule through the two softmaxes gives, for an
// upstream gradient dY,
//   dZ[m]    = sum_n Bt[n][m] dY[n]
//   dV[n]    = sum_m A[m][n] dZ[m]
//   dl[m][n] = A[m][n] (<dZ[m], V[n]> - gam[m]) + Bt[n][m] (<dY[n], Z[m]> - del[n])
//              with gam[m] = <dZ[m], Z[m]>, del[n] = <dY[n], Y[n]>
//   dQ[m]    = s sum_n dl[m][n] K[n]   (summed over the batch: Q is shared)
//   dK[n]    = s sum_m dl[m][n] Q[m].
// Nothing N x M is stored: every kernel recomputes the logits it needs. The
// encode statistics (mu*, sig*) and Z come from the forward's own encode and
// combine; the decode statistics (nu, tau) and del per token from bw_stats.
//
// Layout of work: a pair of lanes (l, l ^ 32) owns one token (token kernels)
// or one latent (latent kernels), each lane holding half of every D-vector;
// dot products add the two halves with one cross-lane swap. All exponentials
// are base 2 on logits scaled by c = s log2(e).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace flare {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) {
    return *p;
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) {
    return __uint_as_float((uint32_t)*p << 16);
}
template <typename T>
__device__ __forceinline__ void st(T* p, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, float v) {
    *p = v;
}
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, float v) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
}

// x summed over the lane pair (l, l ^ 32); the same value in both lanes.
__device__ __forceinline__ float pair_add(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int H2>
__device__ __forceinline__ float half_dot(const float (&a)[H2], const float* b) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < H2; ++i) s = fmaf(a[i], b[i], s);
    return s;
}

constexpr int kTokPerBlock = 128;  // token kernels: 256 threads, a lane pair per token
constexpr int kTile = 64;          // latent kernels: tokens staged per LDS tile

// ---------------------------------------------------------------------------
// Per token: the decode softmax's maximum nu and sum tau (log2 units), and
// del = <dY, Y> = sum_m Bt[n][m] <dY[n], Z[m]>, from a first sweep over the
// latents (running maximum) and a second one (weights against nu).
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void bw_stats(BackwardArgs a) {
    constexpr int H2 = D / 2;
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int lane = threadIdx.x & 63, half = lane >> 5;
    const int n = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6) * 32 + (lane & 31);
    const int N = a.N, M = a.M;
    const int nn = min(n, N - 1);
    const T* Qh = (const T*)a.Q + (int64_t)h * M * D + half * H2;
    const float* Zb = a.Z + (int64_t)bh * M * D + half * H2;
    const T* kr = (const T*)a.K + ((int64_t)bh * N + nn) * D + half * H2;
    const T* gr = (const T*)a.dY + ((int64_t)bh * N + nn) * D + half * H2;
    float k[H2], g[H2];
#pragma unroll
    for (int i = 0; i < H2; ++i) {
        k[i] = ld<T>(kr + i);
        g[i] = ld<T>(gr + i);
    }
    auto logit = [&](int m) {
        float q[H2];
#pragma unroll
        for (int i = 0; i < H2; ++i) q[i] = ld<T>(Qh + (int64_t)m * D + i);
        return a.c * pair_add(half_dot<H2>(q, k));
    };
    float nu = -INFINITY, tau = 0.0f;
    for (int m = 0; m < M; ++m) {
        const float x = logit(m);
        if (x > nu) {
            tau = (nu == -INFINITY) ? 0.0f : tau * exp2f(nu - x);
            nu = x;
        }
        tau += exp2f(x - nu);
    }
    float del = 0.0f;
    for (int m = 0; m < M; ++m) {
        const float w = exp2f(logit(m) - nu);
        del = fmaf(w, pair_add(half_dot<H2>(g, Zb + (int64_t)m * D)), del);
    }
    if (n < N && half == 0) {
        const int64_t o = (int64_t)bh * N + n;
        a.nu[o] = nu;
        a.tau[o] = tau;
        a.del[o] = del / tau;
    }
}

// ---------------------------------------------------------------------------
// Latent kernels: grid (chunks C, B*H, latent groups of 128). The chunk's
// tokens pass through LDS in tiles of 64: K and dY (and V for dQ) as fp32
// rows, with the per-token statistics. A lane pair owns one latent.
// ---------------------------------------------------------------------------
template <int D, typename T, bool DQ>
__global__ __launch_bounds__(256) void bw_latent(BackwardArgs a) {
    constexpr int H2 = D / 2;
    __shared__ float kt[kTile * D], gt[kTile * D], vt[DQ ? kTile * D : 1];
    __shared__ float snu[kTile], stau[kTile], sdel[kTile];
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int chunk = blockIdx.x, bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M;
    const int m = blockIdx.z * 128 + (tid >> 6) * 32 + (lane & 31);
    const int mm = min(m, M - 1);
    const int n0 = chunk * a.chunk_len, n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    float q[H2], zr[H2], dzr[H2], acc[H2];
    const T* qr = (const T*)a.Q + ((int64_t)h * M + mm) * D + half * H2;
#pragma unroll
    for (int i = 0; i < H2; ++i) {
        q[i] = ld<T>(qr + i);
        acc[i] = 0.0f;
        zr[i] = 0.0f;
        dzr[i] = 0.0f;
    }
    float mu = 0.0f, sig = 1.0f, gam = 0.0f;
    if constexpr (DQ) {
        const int64_t r = (int64_t)bh * M + mm;
#pragma unroll
        for (int i = 0; i < H2; ++i) {
            zr[i] = a.Z[r * D + half * H2 + i];
            dzr[i] = a.dZ[r * D + half * H2 + i];
        }
        mu = a.zmu[r];
        sig = a.zsig[r];
        gam = a.gam[r];
    }
    const int64_t tok0 = (int64_t)bh * N;
    for (int t0 = n0; t0 < n1; t0 += kTile) {
        const int nt = min(kTile, n1 - t0);
        for (int e = tid; e < nt * D; e += 256) {
            const int64_t g = (tok0 + t0) * D + e;
            kt[e] = ld<T>((const T*)a.K + g);
            gt[e] = ld<T>((const T*)a.dY + g);
            if constexpr (DQ) vt[e] = ld<T>((const T*)a.V + g);
        }
        for (int e = tid; e < nt; e += 256) {
            snu[e] = a.nu[tok0 + t0 + e];
            stau[e] = a.tau[tok0 + t0 + e];
            sdel[e] = a.del[tok0 + t0 + e];
        }
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const float* kk = kt + t * D + half * H2;
            const float* gg = gt + t * D + half * H2;
            const float x = c * pair_add(half_dot<H2>(q, kk));
            const float bt = exp2f(x - snu[t]) / stau[t];
            if constexpr (!DQ) {
                // dZ[m] += Bt[n][m] dY[n]
#pragma unroll
                for (int i = 0; i < H2; ++i) acc[i] = fmaf(bt, gg[i], acc[i]);
            } else {
                const float* vv = vt + t * D + half * H2;
                const float am = exp2f(x - mu) / sig;
                const float gv = pair_add(half_dot<H2>(dzr, vv));
                const float gy = pair_add(half_dot<H2>(zr, gg));
                const float dl = am * (gv - gam) + bt * (gy - sdel[t]);
#pragma unroll
                for (int i = 0; i < H2; ++i) acc[i] = fmaf(dl, kk[i], acc[i]);
            }
        }
        __syncthreads();
    }
    if (m < M) {
        float* dst = a.part + (((int64_t)bh * gridDim.x + chunk) * M + m) * D + half * H2;
        const float scale = DQ ? a.s : 1.0f;
#pragma unroll
        for (int i = 0; i < H2; ++i) dst[i] = scale * acc[i];
    }
}

// dZ = sum over chunks of the partials, and gam[m] = <dZ[m], Z[m]>.
// One wave per (b, h, m): lane d sums the chunks of column d (all chunks'
// loads in flight together), then the wave reduces gam.
__global__ __launch_bounds__(256) void bw_dz_combine(BackwardArgs a) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // bh * M + m
    const int d = threadIdx.x & 63;
    if (r >= (int64_t)a.BH * a.M) return;
    const int bh = (int)(r / a.M), m = (int)(r - (int64_t)bh * a.M);
    const int D = a.D, C = a.C;
    float s = 0.0f, gz = 0.0f;
    if (d < D) {
        const float* p = a.part + ((int64_t)bh * C * a.M + m) * D + d;
        const int64_t step = (int64_t)a.M * D;
        for (int ch = 0; ch < C; ++ch) s += p[ch * step];
        a.dZ[r * D + d] = s;
        gz = s * a.Z[r * D + d];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gz += __shfl_xor(gz, off, 64);
    if (d == 0) a.gam[r] = gz;
}

// dQ[h] = sum over the batch and the chunks of the partials (already scaled
// by s), stored in the operator dtype. One thread per (h, m, d).
template <typename T>
__global__ __launch_bounds__(256) void bw_dq_combine(BackwardArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (h * M + m) * D + d
    const int64_t MD = (int64_t)a.M * a.D;
    if (e >= (int64_t)a.H * MD) return;
    const int h = (int)(e / MD);
    const int64_t md = e - (int64_t)h * MD;
    const int B = a.BH / a.H, C = a.C;
    float s = 0.0f;
    for (int b = 0; b < B; ++b)
        for (int ch = 0; ch < C; ++ch) s += a.part[((int64_t)(b * a.H + h) * C + ch) * MD + md];
    st<T>((T*)a.dQ + e, s);
}

// ---------------------------------------------------------------------------
// Per token: dV[n] = sum_m A[m][n] dZ[m] and dK[n] = s sum_m dl[m][n] Q[m].
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void bw_dkdv(BackwardArgs a) {
    constexpr int H2 = D / 2;
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int lane = threadIdx.x & 63, half = lane >> 5;
    const int n = blockIdx.x * kTokPerBlock + (threadIdx.x >> 6) * 32 + (lane & 31);
    const int N = a.N, M = a.M;
    const int nn = min(n, N - 1);
    const int64_t row = ((int64_t)bh * N + nn) * D + half * H2;
    float k[H2], v[H2], g[H2], dk[H2], dv[H2];
#pragma unroll
    for (int i = 0; i < H2; ++i) {
        k[i] = ld<T>((const T*)a.K + row + i);
        v[i] = ld<T>((const T*)a.V + row + i);
        g[i] = ld<T>((const T*)a.dY + row + i);
        dk[i] = 0.0f;
        dv[i] = 0.0f;
    }
    const int64_t o = (int64_t)bh * N + nn;
    const float nu = a.nu[o], rtau = 1.0f / a.tau[o], del = a.del[o];
    const T* Qh = (const T*)a.Q + (int64_t)h * M * D + half * H2;
    const int64_t zoff = (int64_t)bh * M;
    for (int m = 0; m < M; ++m) {
        float q[H2];
#pragma unroll
        for (int i = 0; i < H2; ++i) q[i] = ld<T>(Qh + (int64_t)m * D + i);
        const float* zr = a.Z + (zoff + m) * D + half * H2;
        const float* dzr = a.dZ + (zoff + m) * D + half * H2;
        const float x = a.c * pair_add(half_dot<H2>(q, k));
        const float am = exp2f(x - a.zmu[zoff + m]) / a.zsig[zoff + m];
        const float bt = exp2f(x - nu) * rtau;
        const float gv = pair_add(half_dot<H2>(v, dzr));
        const float gy = pair_add(half_dot<H2>(g, zr));
        const float dl = am * (gv - a.gam[zoff + m]) + bt * (gy - del);
#pragma unroll
        for (int i = 0; i < H2; ++i) {
            dk[i] = fmaf(dl, q[i], dk[i]);
            dv[i] = fmaf(am, dzr[i], dv[i]);
        }
    }
    if (n < N) {
#pragma unroll
        for (int i = 0; i < H2; ++i) {
            st<T>((T*)a.dK + row + i, a.s * dk[i]);
            st<T>((T*)a.dV + row + i, dv[i]);
        }
    }
}

#define FLARE_BW_DISPATCH(FN, a, s)      \
    switch ((a).D) {                     \
        case 8: return FN<8>(a, s);      \
        case 16: return FN<16>(a, s);    \
        case 24: return FN<24>(a, s);    \
        case 32: return FN<32>(a, s);    \
        case 48: return FN<48>(a, s);    \
        case 64: return FN<64>(a, s);    \
        default: return hipErrorInvalidValue; \
    }

template <int D>
hipError_t stats_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid((a.N + kTokPerBlock - 1) / kTokPerBlock, a.BH);
    if (a.bf16)
        hipLaunchKernelGGL((bw_stats<D, uint16_t>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bw_stats<D, float>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t dz_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH, (a.M + 127) / 128);
    if (a.bf16)
        hipLaunchKernelGGL((bw_latent<D, uint16_t, false>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bw_latent<D, float, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t dq_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH, (a.M + 127) / 128);
    if (a.bf16)
        hipLaunchKernelGGL((bw_latent<D, uint16_t, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bw_latent<D, float, true>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t dkdv_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid((a.N + kTokPerBlock - 1) / kTokPerBlock, a.BH);
    if (a.bf16)
        hipLaunchKernelGGL((bw_dkdv<D, uint16_t>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((bw_dkdv<D, float>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool backward_supports(int D) { return D == 8 || D == 16 || D == 24 || D == 32 || D == 48 || D == 64; }

hipError_t launch_bw_stats(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(stats_d, a, s) }
hipError_t launch_bw_dz(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(dz_d, a, s) }
hipError_t launch_bw_dq(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(dq_d, a, s) }
hipError_t launch_bw_dkdv(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(dkdv_d, a, s) }

hipError_t launch_bw_dz_combine(const BackwardArgs& a, hipStream_t s) {
    const int64_t n = (int64_t)a.BH * a.M;  // one wave each, four per workgroup
    hipLaunchKernelGGL(bw_dz_combine, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bw_dq_combine(const BackwardArgs& a, hipStream_t s) {
    const int64_t n = (int64_t)a.H * a.M * a.D;
    if (a.bf16)
        hipLaunchKernelGGL(bw_dq_combine<uint16_t>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(bw_dq_combine<float>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace flare
