// Backward of the FLARE forward (gradients of Q, K and V): fp32 VALU kernels
// (any supported storage, D <= 64) and, for bf16 heads whose Q, Z and dZ fit in
// LDS, matrix-core kernels (bw_stats_bf16, bw_dkdv_bf16, bw_lat_bf16).
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
// The dZ and dQ partial sums come from the latent kernels, or (bf16, D = 32,
// M <= 128) from the token-side kernels themselves: dZ from bw_stats_bf16,
// dQ from bw_dkdv_bf16.
//
// Layout of work in the fp32 kernels: a pair of lanes (l, l ^ 32) owns one
// token (token kernels) or one latent (latent kernels), each lane holding half
// of every D-vector; dot products add the two halves with one cross-lane swap.
// All exponentials are base 2 on logits scaled by c = s log2(e).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "launch.h"

namespace flare {
namespace {

#include "gfx950_ops.h"

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

// Element offset of head bh's token 0 in K, V, dY, dK and dV (token rows
// are a.sn elements apart: D in the [B][H][N][D] layout, H * D in the
// token-major [B][N][H][D] one).
__device__ __forceinline__ int64_t head_base(const BackwardArgs& a, int bh) {
    const int b = bh / a.H;
    return b * a.sb + (bh - b * a.H) * a.sh;
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
    const int64_t row = head_base(a, bh) + nn * a.sn + half * H2;
    const T* kr = (const T*)a.K + row;
    const T* gr = (const T*)a.dY + row;
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
// tokens pass through LDS in tiles of 64 (32 above D = 64): K and dY (and V
// for dQ) as fp32 rows, with the per-token statistics. A lane pair owns one
// latent.
// ---------------------------------------------------------------------------
template <int D, typename T, bool DQ>
__global__ __launch_bounds__(256) void bw_latent(BackwardArgs a) {
    constexpr int H2 = D / 2, TL = D > 64 ? kTile / 2 : kTile;  // at most 48 KB of tiles
    __shared__ float kt[TL * D], gt[TL * D], vt[DQ ? TL * D : 1];
    __shared__ float snu[TL], stau[TL], sdel[TL];
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
    const int64_t tok0 = (int64_t)bh * N, hb = head_base(a, bh);
    for (int t0 = n0; t0 < n1; t0 += TL) {
        const int nt = min(TL, n1 - t0);
        for (int e = tid; e < nt * D; e += 256) {
            const int64_t g = hb + (t0 + e / D) * a.sn + e % D;
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
// One wave per (b, h, m): lane d sums the chunks of columns d, d + 64, ...
// (all chunks' loads in flight together), then the wave reduces gam.
__global__ __launch_bounds__(256) void bw_dz_combine(BackwardArgs a) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // bh * M + m
    const int lane = threadIdx.x & 63;
    if (r >= (int64_t)a.BH * a.M) return;
    const int bh = (int)(r / a.M), m = (int)(r - (int64_t)bh * a.M);
    const int D = a.D, C = a.C;
    float gz = 0.0f;
    for (int d = lane; d < D; d += 64) {
        float s = 0.0f;
        const float* p = a.part + ((int64_t)bh * C * a.M + m) * D + d;
        const int64_t step = (int64_t)a.M * D;
        for (int ch = 0; ch < C; ++ch) s += p[ch * step];
        a.dZ[r * D + d] = s;
        gz = fmaf(s, a.Z[r * D + d], gz);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gz += __shfl_xor(gz, off, 64);
    if (lane == 0) a.gam[r] = gz;
}

// dQ[h] = sum over the batch and the chunks of the partials (already scaled
// by s), stored in the operator dtype. A workgroup covers 64 consecutive
// entries (h, m, d); its four waves sum interleaved quarters of the B * C
// partials, which are then added in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void bw_dq_combine(BackwardArgs a) {
    __shared__ float red[3][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.x * 64 + lane;  // (h * M + m) * D + d
    const int64_t MD = (int64_t)a.M * a.D;
    const bool in = e < (int64_t)a.H * MD;
    float s = 0.0f;
    if (in) {
        const int h = (int)(e / MD);
        const int64_t md = e - (int64_t)h * MD;
        const int B = a.BH / a.H, C = a.C;
        for (int q = w; q < B * C; q += 4) {
            const int b = q / C, ch = q - b * C;
            s += a.part[((int64_t)(b * a.H + h) * C + ch) * MD + md];
        }
    }
    if (w > 0) red[w - 1][lane] = s;
    __syncthreads();
    if (w == 0 && in) st<T>((T*)a.dQ + e, s + red[0][lane] + red[1][lane] + red[2][lane]);
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
    const int64_t row = head_base(a, bh) + nn * a.sn + half * H2;
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
            // accum: added to what dK, dV hold (fp32 sum, rounded once)
            const float k0 = a.accum ? ld<T>((const T*)a.dK + row + i) : 0.0f;
            const float v0 = a.accum ? ld<T>((const T*)a.dV + row + i) : 0.0f;
            st<T>((T*)a.dK + row + i, k0 + a.s * dk[i]);
            st<T>((T*)a.dV + row + i, v0 + dv[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward on the matrix core (bf16 storage; see the backward notes in
// kernels_backward.hip for the formulas). Token-parallel like the decode: a
// wave owns 32 tokens and walks the latents in blocks of 32; the head's Q, Z
// and dZ rows sit in LDS as bf16 (natural latent order, swizzled rows).
// ---------------------------------------------------------------------------
// Stage rows [Mp][D] of a matrix (bf16 storage, or fp32 rounded to nearest
// even) into a swizzled LDS tile; rows >= M are zero.
template <int D, typename ST>
__device__ __forceinline__ void stage_rows(unsigned char* dst, const ST* src, int M, int Mp, int tid, int nth) {
    constexpr int CH = D / 8;
    for (int p = tid; p < Mp * CH; p += nth) {
        const int m = p / CH, ch = p % CH;
        bf16x8 v = zero8();
        if (m < M) {
            if constexpr (sizeof(ST) == 4) {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (__bf16)(float)src[(int64_t)m * D + ch * 8 + j];
            } else {
                v = *(const bf16x8*)(src + (int64_t)m * D + ch * 8);
            }
        }
        *(bf16x8*)(dst + tile_off<D>(m, ch)) = v;
    }
}

// Per token: nu' = log2-sum-exp2 of the logits over the latents (the decode
// softmax's normaliser, log2 units) and del = <dY, Y> = sum_m Bt[n][m] <dY[n],
// Z[m]>. One sweep over the latents against a bound on every logit of the
// head, with a second against the token's exact maximum where the first
// underflows. FDZ (D = 32 with M <= 128, or D = 64 with M <= 64): a further
// sweep forms Bt and the dZ partial sums, dZ^T[d][m] += dY^T[d][n] Bt[n][m]
// over the workgroup's tokens.
template <int D, bool FDZ = false>
__global__ __launch_bounds__(256) void bw_stats_bf16(BackwardArgs a) {
    static_assert(!FDZ || D == 32 || D == 64, "dZ fused at D = 32 or 64 only");
    constexpr int KB = D / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char bsm[];
    const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = (M + 31) & ~31, MB = Mp / 32;
    const float c = a.c;
    unsigned char* qs = bsm;
    unsigned char* zs = bsm + Mp * 2 * D;
    stage_rows<D>(qs, (const uint16_t*)a.Q + (int64_t)h * M * D, M, Mp, tid, 256);
    stage_rows<D>(zs, a.Z + (int64_t)bh * M * D, M, Mp, tid, 256);
    // One offset for the head: every logit satisfies c l <= mu*[m] + 32 (each
    // tile the forward's encode accepted had probabilities <= 2^32 against
    // its running offset, and mu* is the largest of those), so 2^(c l - nub)
    // <= 1 everywhere; a token whose sum falls below 2^-90 is redone against
    // its exact maximum.
    float* red = (float*)(zs + Mp * 2 * D);
    // FDZ (dZ fused in): this wave's dY rows of the block, scaled by the
    // token's 1/tau (zero past N), and its tiles [token][latent] of the
    // sweep's weights 2^(c l - nu) for each latent block, bf16 rows
    // (swizzled); the head's dZ^T sums over this wave's tokens stay in
    // registers, for up to MBX latent blocks
    constexpr int DB = D / 32, MBX = 4 / DB, MBU = FDZ ? MBX : 1;  // 64 accumulator registers
    unsigned char* gtile = (unsigned char*)(red + 4) + wave * (32 * 2 * D + MBX * 32 * 64);
    unsigned char* btile = gtile + 32 * 2 * D;
    f32x16 dz[FDZ ? MBX : 1][DB];
#pragma unroll
    for (int j = 0; j < (FDZ ? MBX : 1); ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) dz[j][db] = f32x16{};
    const int g = lane >> 4, gi = lane & 15;
    float mz = -INFINITY;
    for (int m = tid; m < M; m += 256) mz = fmaxf(mz, a.zmu[(int64_t)bh * M + m]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mz = fmaxf(mz, __shfl_xor(mz, off, 64));
    if (lane == 0) red[wave] = mz;
    __syncthreads();
    const float nub = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) + 32.0f;
    const int64_t sn = a.sn;
    const uint16_t* Kb = (const uint16_t*)a.K + head_base(a, bh);
    const uint16_t* Gb = (const uint16_t*)a.dY + head_base(a, bh);
    const int nblk = (N + 31) / 32, bstep = gridDim.x * 4;
    int blk = blockIdx.x * 4 + wave;
    if (!FDZ && blk >= nblk) return;  // no barrier follows (FDZ: the waves merge at the end)
    // this block's K and dY rows; the next block's are loaded while this one
    // is processed (clamped to the last block, so the loads are unconditional
    // and the compiler's wait before the first use covers exactly them)
    bf16x8 kop[KB], gop[KB], kpf[KB], gpf[KB];
    auto load = [&](int bk, bf16x8(&ko)[KB], bf16x8(&go)[KB]) {
        const int nn = min(bk * 32 + l32, N - 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            ko[kb] = *(const bf16x8*)(Kb + nn * sn + 16 * kb + 8 * hi);
            go[kb] = *(const bf16x8*)(Gb + nn * sn + 16 * kb + 8 * hi);
        }
    };
    load(min(blk, nblk - 1), kpf, gpf);
    auto rows = [&](const unsigned char* t, int mb, bf16x8 (&op)[KB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) op[kb] = *(const bf16x8*)(t + tile_off<D>(32 * mb + l32, 2 * kb + hi));
    };
    // register i holds latent 32 mb + 8 (i/4) + 4 hi + i%4 (natural rows);
    // only the last block can hold padding rows
    auto valid = [&](int mb, int i) { return 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3) < M; };
    const bool padded = M != Mp;
    for (; blk < nblk; blk += bstep) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kop[kb] = kpf[kb];
            gop[kb] = gpf[kb];
        }
        load(min(blk + bstep, nblk - 1), kpf, gpf);
        // sums of 2^(c l - nu) and of those weights times <dY, Z[m]>; FDZ:
        // the weights also go to the wave's tiles, rounded to bf16 (register
        // i: latent 32 mb + 8 (i/4) + 4 hi + i%4 -> 8 bytes per 4)
        auto sweep = [&](float nu, float& tau, float& pg) {
            tau = 0.0f;
            pg = 0.0f;
            for (int mb = 0; mb < MB; ++mb) {
                bf16x8 qa[KB], za[KB];
                rows(qs, mb, qa);
                rows(zs, mb, za);
                f32x16 S = mfma(qa[0], kop[0], f32x16{});
                f32x16 G = mfma(za[0], gop[0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) {
                    S = mfma(qa[kb], kop[kb], S);
                    G = mfma(za[kb], gop[kb], G);
                }
                float p[16];
                if (padded && mb == MB - 1) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) p[i] = valid(mb, i) ? exp2_fast(fmaf(S[i], c, -nu)) : 0.0f;
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) p[i] = exp2_fast(fmaf(S[i], c, -nu));
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    tau += p[i];
                    pg = fmaf(p[i], G[i], pg);
                }
                if constexpr (FDZ) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16x2 w01 = {(__bf16)p[4 * q], (__bf16)p[4 * q + 1]};
                        const bf16x2 w23 = {(__bf16)p[4 * q + 2], (__bf16)p[4 * q + 3]};
                        const u32x2 w = {__builtin_bit_cast(uint32_t, w01), __builtin_bit_cast(uint32_t, w23)};
                        *(u32x2*)(btile + mb * (32 * 64) + tile_off<32>(l32, q) + 8 * hi) = w;
                    }
                }
            }
            tau = pair_sum(tau);
            pg = pair_sum(pg);
        };
        float nu = nub, tau, pg;
        sweep(nu, tau, pg);
        if (wave_any(!(tau >= 8.077935669463161e-28f))) {  // 2^-90: redo against the exact maxima
            float mx = -INFINITY;
            for (int mb = 0; mb < MB; ++mb) {
                bf16x8 qa[KB];
                rows(qs, mb, qa);
                f32x16 S = mfma(qa[0], kop[0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) S = mfma(qa[kb], kop[kb], S);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (valid(mb, i)) mx = fmaxf(mx, S[i]);
            }
            nu = pair_max(mx) * c;
            sweep(nu, tau, pg);
        }
        // every lane stores (both lanes of a token hold the same sums, and
        // lanes past N repeat token N - 1's values), so the stores are
        // unconditional and the next wait stays exact
        const int64_t o = (int64_t)bh * N + min(blk * 32 + l32, N - 1);
        const float nup = nu + __log2f(tau);
        a.nu[o] = nup;  // with tau = 1: the weights are normalised by nu alone
        a.tau[o] = 1.0f;
        a.del[o] = pg / tau;
        if constexpr (FDZ) {
            // dZ^T[d][m] += sum over tokens dY^T[d][n] Bt[n][m], with
            // Bt[n][m] = 2^(c l - nu') = 2^(c l - nu) / tau: the sweep's
            // weights are in the tiles, and the token's 1/tau goes with its
            // dY row (rounded to bf16 once scaled). Transposed reads of the
            // tiles give dY^T (rows d, k = tokens) and the weights (k =
            // tokens, columns = latents); padding latents have weight 0.
            // W: the tile's row width in bf16 (D for dY, 32 latents for Bt)
            auto tr_addr = [&](auto W, const unsigned char* t, int kp, int db, int second) {
                const int row = 16 * kp + 8 * (g >> 1) + (gi >> 2) + 4 * second;
                const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
                return t + tile_off<decltype(W)::value>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
            };
            const std::integral_constant<int, D> wd;
            const std::integral_constant<int, 32> wb;
            const int n = blk * 32 + l32;
            const float rt = 1.0f / tau;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                bf16x8 v = zero8();
                if (n < N) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = (__bf16)((float)gop[kb][j] * rt);
                }
                *(bf16x8*)(gtile + tile_off<D>(l32, 2 * kb + hi)) = v;
            }
            bf16x8 gt[2][DB];
#pragma unroll
            for (int db = 0; db < DB; ++db)
                lds_tr_op2_c(tr_addr(wd, gtile, 0, db, 0), tr_addr(wd, gtile, 0, db, 1), tr_addr(wd, gtile, 1, db, 0),
                             tr_addr(wd, gtile, 1, db, 1), gt[0][db], gt[1][db]);
#pragma unroll MBU
            for (int mb = 0; mb < MBX; ++mb) {
                if (mb >= MB) continue;
                const unsigned char* bt = btile + mb * (32 * 64);
                bf16x8 bt0, bt1;
                lds_tr_op2_c(tr_addr(wb, bt, 0, 0, 0), tr_addr(wb, bt, 0, 0, 1), tr_addr(wb, bt, 1, 0, 0),
                             tr_addr(wb, bt, 1, 0, 1), bt0, bt1);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dz[mb][db] = mfma(gt[0][db], bt0, dz[mb][db]);
                    dz[mb][db] = mfma(gt[1][db], bt1, dz[mb][db]);
                }
            }
        }
    }
    if constexpr (FDZ) {
        // merge the four waves' dZ^T sums (fixed order) and write this
        // workgroup's partial: slot blockIdx.x of [BH][gridDim.x][M][D].
        // Register r of accumulator (j, db): d = 32 db + 8 (r/4) + 4 hi + r%4,
        // latent 32 j + l32.
        __syncthreads();  // staged rows and tiles are no longer read
        float* mbuf = (float*)bsm;
        constexpr int PER = MBX * DB * 16 * 64;
        if (wave > 0) {
            float* d0 = mbuf + (wave - 1) * PER;
#pragma unroll
            for (int j = 0; j < MBX; ++j)
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) d0[((j * DB + db) * 16 + r) * 64 + lane] = dz[j][db][r];
        }
        __syncthreads();
        if (wave == 0) {
            for (int t = 0; t < 3; ++t) {
                const float* s0 = mbuf + t * PER;
#pragma unroll
                for (int j = 0; j < MBX; ++j)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) dz[j][db][r] += s0[((j * DB + db) * 16 + r) * 64 + lane];
            }
#pragma unroll
            for (int j = 0; j < MBX; ++j) {
                const int m = 32 * j + l32;
                if (j < MB && m < M) {
                    float* dst = a.part + (((int64_t)bh * gridDim.x + blockIdx.x) * M + m) * D;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const f32x4 v = {dz[j][db][4 * g4], dz[j][db][4 * g4 + 1], dz[j][db][4 * g4 + 2],
                                             dz[j][db][4 * g4 + 3]};
                            *(f32x4*)(dst + 32 * db + 8 * g4 + 4 * hi) = v;
                        }
                }
            }
        }
    }
}

// Per token: dV[n] = sum_m A[m][n] dZ[m] and dK[n] = s sum_m dl[m][n] Q[m].
// The A operands of the three logit-shaped products (Q K^T, Z dY^T, dZ V^T)
// take latent rows in the order enc_row_token gives, so that registers
// 8 kp .. 8 kp + 7 of a lane hold latents 32 mb + 16 kp + 8 hi + 0..7, which
// are exactly the k-slots of the B operand of the accumulations dK^T += Q^T dl
// and dV^T += dZ^T A, whose A operands are read transposed from the natural
// row-major LDS rows.
// FDQ (bf16, M <= 32 MBX: 128 at D = 32, 64 at D = 64): the same kernel
// also forms dQ's partial sums, dQ^T[d][m] += K^T[d][n] dl[m][n] over the
// workgroup's tokens, so that no separate latent-side pass over K, V and dY
// is needed for dQ.

// ENC: the encode's backward alone (first stage of the FLARE++ backward):
// dl = A (dZ V^T - gam), no decode weights, no dY.
// NWV: waves per workgroup. Eight at D = 64 with more than 128 latents
// (without FDQ): the head's Q, Z and dZ rows (96 KB at M = 256) then feed two
// waves per SIMD from one LDS copy, at most 256 registers each (no prefetch of
// the next block's rows; the other wave hides the loads). Measured on MI355X:
// 3% faster on the large mesh (M = 256), 2% slower at M = 128.
template <int D, bool ENC = false, bool FDQ = false, int MBX = 4, int NWV = 4>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu((FDQ && D == 32) || NWV == 8 ? 2 : 1))) void bw_dkdv_bf16(
    BackwardArgs a) {
    static_assert(!(FDQ && ENC), "dQ fused with the full formula only");
    static_assert(NWV == 4 || (NWV == 8 && !FDQ), "the dQ merge is written for four waves");
    constexpr int NT = 64 * NWV;
    constexpr int KB = D / 16, DB = D / 32;
    // the -del start of the Z dY^T products is a 16-register broadcast held
    // through the latent loop: not in the eight-wave form, which has no
    // registers to spare, nor at D = 128
    constexpr bool kDelInit = NWV == 4 && D != 128;
    extern __shared__ __attribute__((aligned(16))) unsigned char bsm[];
    const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = (M + 31) & ~31, MB = Mp / 32;
    const float c = a.c;
    unsigned char* qs = bsm;
    unsigned char* zs = qs + Mp * 2 * D;               // Z rows (not with ENC)
    unsigned char* dzs = zs + (ENC ? 0 : Mp * 2 * D);
    float* lam = (float*)(dzs + Mp * 2 * D);  // [Mp] mu* + log2 sig* (+inf for padding)
    float* gam = lam + Mp;                     // [Mp] -gam (negated: the dZ V^T products start from it)
    float* sbias = gam + Mp;                   // [Mp] 0, or -1e30 for padding (the logits' start)
    // FDQ (dQ fused in): this wave's K rows of the block (zero past N) and
    // its dl tile [token][latent] of the current latent block, bf16 rows
    // (swizzled); the head's dQ^T sums over this wave's tokens stay in
    // registers, for up to MBX latent blocks
    unsigned char* ktile = (unsigned char*)(sbias + Mp) + wave * (32 * 2 * D + 32 * 64);
    unsigned char* ptile = ktile + 32 * 2 * D;
    constexpr int MBU = FDQ ? MBX : 1;
    f32x16 dq[FDQ ? MBX : 1][DB];
#pragma unroll
    for (int j = 0; j < (FDQ ? MBX : 1); ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) dq[j][db] = f32x16{};
    stage_rows<D>(qs, (const uint16_t*)a.Q + (int64_t)h * M * D, M, Mp, tid, NT);
    if constexpr (!ENC) stage_rows<D>(zs, a.Z + (int64_t)bh * M * D, M, Mp, tid, NT);
    stage_rows<D>(dzs, a.dZ + (int64_t)bh * M * D, M, Mp, tid, NT);
    for (int m = tid; m < Mp; m += NT) {
        const int64_t r = (int64_t)bh * M + m;
        lam[m] = m < M ? a.zmu[r] + __log2f(a.zsig[r]) : INFINITY;
        gam[m] = m < M ? -a.gam[r] : 0.0f;
        sbias[m] = m < M ? 0.0f : -1e30f;
    }
    __syncthreads();
    const int64_t sn = a.sn, hb = head_base(a, bh);
    const uint16_t* Kb = (const uint16_t*)a.K + hb;
    const uint16_t* Vb = (const uint16_t*)a.V + hb;
    const uint16_t* Gb = (const uint16_t*)a.dY + hb;
    const int g = lane >> 4, gi = lane & 15;
    const int prow = enc_row_token(l32);
    const int nblk = (N + 31) / 32, bstep = gridDim.x * NWV;
    const bool padded = M != Mp;
    int blk = blockIdx.x * NWV + wave;
    if (!FDQ && blk >= nblk) return;  // no barrier follows (FDQ: the waves merge at the end)
    // this block's K, V (and dY) rows and per-token statistics; the next
    // block's are loaded while this one is processed (clamped to the last
    // block, so the loads are unconditional and the compiler's wait before
    // the first use covers exactly them)
    // (FDQ holds its dQ sums in the registers a second set would take (at
    // D = 32 at two waves per SIMD; at D = 64 prefetching there measured 4%
    // slower): there each block's rows are loaded at its start)
    constexpr bool PF = !FDQ && NWV == 4 && D != 128;  // (D = 128: 460 registers without, no spills)
    bf16x8 kop[KB], vop[KB], gop[KB], kpf[KB], vpf[KB], gpf[KB];
    float nu, del, nupf = 0.0f, delpf = 0.0f;
    auto load = [&](int bk) {
        const int nn = min(bk * 32 + l32, N - 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t o = nn * sn + 16 * kb + 8 * hi;
            kpf[kb] = *(const bf16x8*)(Kb + o);
            vpf[kb] = *(const bf16x8*)(Vb + o);
            if constexpr (!ENC) gpf[kb] = *(const bf16x8*)(Gb + o);
        }
        if constexpr (!ENC) {
            nupf = a.nu[(int64_t)bh * N + nn];
            delpf = a.del[(int64_t)bh * N + nn];
        }
    };
    if constexpr (PF) load(blk);
    for (; blk < nblk; blk += bstep) {
        const int n = blk * 32 + l32, nn = min(n, N - 1);
        if constexpr (!PF) load(blk);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kop[kb] = kpf[kb];
            vop[kb] = vpf[kb];
            if constexpr (!ENC) gop[kb] = gpf[kb];
        }
        nu = nupf;
        del = delpf;
        if constexpr (PF) load(min(blk + bstep, nblk - 1));
        f32x16 ndel;
        if constexpr (kDelInit) {
#pragma unroll
            for (int r = 0; r < 16; ++r) ndel[r] = -del;
        }
        // ENC with accum: this block's old dK and dV (the second stage's
        // gradients), in the store layout, requested now so that their
        // latency overlaps the block's work
        u32x2 okr[ENC ? DB : 1][4], ovr[ENC ? DB : 1][4];
        if constexpr (ENC) {
            if (a.accum) {
                const uint16_t* oK = (const uint16_t*)a.dK + hb + nn * sn;
                const uint16_t* oV = (const uint16_t*)a.dV + hb + nn * sn;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d0 = 32 * db + 8 * g4 + 4 * hi;
                        okr[db][g4] = *(const u32x2*)(oK + d0);
                        ovr[db][g4] = *(const u32x2*)(oV + d0);
                    }
            }
        }
        f32x16 dk[DB], dv[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            dk[db] = f32x16{};
            dv[db] = f32x16{};
        }
        // FDQ: K^T operands of this block (rows d, k = tokens), transposed
        // reads of the K tile; rows past N are zero, so their dl adds nothing
        // (W: the tile's row width in elements, D for K rows, 32 for dl rows)
        auto tr_addr = [&](auto W, const unsigned char* t, int row0, int kp, int db, int second) {
            const int row = row0 + 16 * kp + 8 * (g >> 1) + (gi >> 2) + 4 * second;
            const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
            return t + tile_off<decltype(W)::value>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
        };
        const std::integral_constant<int, D> WK{};
        const std::integral_constant<int, 32> WP{};
        bf16x8 kt[2][DB];
        if constexpr (FDQ) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                *(bf16x8*)(ktile + tile_off<D>(l32, 2 * kb + hi)) = n < N ? kop[kb] : zero8();
#pragma unroll
            for (int db = 0; db < DB; ++db)
                lds_tr_op2_c(tr_addr(WK, ktile, 0, 0, db, 0), tr_addr(WK, ktile, 0, 0, db, 1),
                             tr_addr(WK, ktile, 0, 1, db, 0), tr_addr(WK, ktile, 0, 1, db, 1), kt[0][db], kt[1][db]);
        }
        // (FDQ: unrolled, so that each latent block's dQ sums stay in registers)
#pragma unroll MBU
        for (int mb = 0; mb < (FDQ ? MBX : MB); ++mb) {
            if (FDQ && mb >= MB) continue;
            f32x16(&dqb)[DB] = dq[FDQ ? mb : 0];
            bf16x8 qa[KB], za[KB], dza[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = tile_off<D>(32 * mb + prow, 2 * kb + hi);
                qa[kb] = *(const bf16x8*)(qs + off);
                if constexpr (!ENC) za[kb] = *(const bf16x8*)(zs + off);
                dza[kb] = *(const bf16x8*)(dzs + off);
            }
            // The dZ V^T products start from -gam of their latents (and,
            // with kDelInit, the Z dY^T products from -del of the token), so
            // that the matrix core leaves dZ.V - gam (and dY.Z - del):
            // register 8 kp + j of a lane holds latent 32 mb + 16 kp + 8 hi + j
            // of token l32. The logits of padded latents (zero rows, last
            // block only) start from -1e30, so that both their weights are 0:
            // the decode weight 2^(c l - nu) of a zero row would otherwise
            // overflow where nu < -128, and the dK sum over the latents would
            // take its inf times the zero Q row.
            auto rowvec = [&](const float* t) __attribute__((always_inline)) {
                f32x16 v;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 x = *(const f32x4*)(t + 32 * mb + 16 * (q >> 1) + 8 * hi + 4 * (q & 1));
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
                }
                return v;
            };
            f32x16 s0 = f32x16{};
            if (!ENC && padded && mb == MB - 1) s0 = rowvec(sbias);
            f32x16 S = mfma(qa[0], kop[0], s0);
            f32x16 GV = mfma(dza[0], vop[0], rowvec(gam));
            f32x16 GY;
            if constexpr (!ENC) GY = mfma(za[0], gop[0], kDelInit ? ndel : f32x16{});
#pragma unroll
            for (int kb = 1; kb < KB; ++kb) {
                S = mfma(qa[kb], kop[kb], S);
                if constexpr (!ENC) GY = mfma(za[kb], gop[kb], GY);
                GV = mfma(dza[kb], vop[kb], GV);
            }
            bf16x8 pe[2], pl[2];
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
                const int m0 = 32 * mb + 16 * kp + 8 * hi;
                const f32x4 l0 = *(const f32x4*)(lam + m0), l1 = *(const f32x4*)(lam + m0 + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 8 * kp + j;
                    const float lj = j < 4 ? l0[j] : l1[j - 4];
                    const float p_e = exp2_fast(fmaf(S[i], c, -lj));
                    float dl = p_e * GV[i];
                    if constexpr (!ENC) dl = fmaf(exp2_fast(fmaf(S[i], c, -nu)), kDelInit ? GY[i] : GY[i] - del, dl);
                    pe[kp][j] = (__bf16)p_e;
                    pl[kp][j] = (__bf16)dl;
                }
            }
            // Q^T and dZ^T operands (rows d, k = latents of this block),
            // transposed reads of the natural rows
            auto taddr = [&](const unsigned char* t, int kp, int db, int second) {
                const int row = 32 * mb + 16 * kp + 8 * (g >> 1) + (gi >> 2) + 4 * second;
                const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
                return t + tile_off<D>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
            };
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x8 qt0, qt1, zt0, zt1;
                lds_tr_op2_c(taddr(qs, 0, db, 0), taddr(qs, 0, db, 1), taddr(qs, 1, db, 0), taddr(qs, 1, db, 1), qt0,
                             qt1);
                lds_tr_op2_c(taddr(dzs, 0, db, 0), taddr(dzs, 0, db, 1), taddr(dzs, 1, db, 0), taddr(dzs, 1, db, 1),
                             zt0, zt1);
                dk[db] = mfma(qt0, pl[0], dk[db]);
                dk[db] = mfma(qt1, pl[1], dk[db]);
                dv[db] = mfma(zt0, pe[0], dv[db]);
                dv[db] = mfma(zt1, pe[1], dv[db]);
            }
            if constexpr (FDQ) {
                // dQ^T[d][m] += sum over tokens K^T[d][n] dl[m][n]: dl goes
                // through the wave's tile [token][latent] (pl[kp] holds
                // latents 16 kp + 8 hi + 0..7 of token l32), and transposed
                // reads give the B operands (k = tokens, columns = latents)
                *(bf16x8*)(ptile + tile_off<32>(l32, hi)) = pl[0];
                *(bf16x8*)(ptile + tile_off<32>(l32, 2 + hi)) = pl[1];
                bf16x8 pt0, pt1;
                lds_tr_op2_c(tr_addr(WP, ptile, 0, 0, 0, 0), tr_addr(WP, ptile, 0, 0, 0, 1),
                             tr_addr(WP, ptile, 0, 1, 0, 0), tr_addr(WP, ptile, 0, 1, 0, 1), pt0, pt1);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dqb[db] = mfma(kt[0][db], pt0, dqb[db]);
                    dqb[db] = mfma(kt[1][db], pt1, dqb[db]);
                }
            }
        }
        // register r of lane l: d = 32 db + 8 (r/4) + 4 hi + r%4, token l32
        // every lane stores: lanes past N repeat token N - 1's rows and
        // values, so the stores are unconditional and the next wait stays
        // exact
        {
            uint16_t* dK = (uint16_t*)a.dK + hb + nn * sn;
            uint16_t* dV = (uint16_t*)a.dV + hb + nn * sn;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d0 = 32 * db + 8 * g4 + 4 * hi;
                    u32x2 wk, wv;
                    float k[4], v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        k[j] = a.s * dk[db][4 * g4 + j];
                        v[j] = dv[db][4 * g4 + j];
                    }
                    if (a.accum) {  // added to what dK, dV hold (fp32 sum, rounded once)
                        u32x2 ok, ov;
                        if constexpr (ENC) {
                            ok = okr[db][g4];
                            ov = ovr[db][g4];
                        } else {
                            ok = *(const u32x2*)(dK + d0);
                            ov = *(const u32x2*)(dV + d0);
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t wk0 = ok[j >> 1], wv0 = ov[j >> 1];
                            k[j] += __uint_as_float((j & 1) ? (wk0 & 0xffff0000u) : (wk0 << 16));
                            v[j] += __uint_as_float((j & 1) ? (wv0 & 0xffff0000u) : (wv0 << 16));
                        }
                    }
                    const bf16x2 k01 = {(__bf16)k[0], (__bf16)k[1]};
                    const bf16x2 k23 = {(__bf16)k[2], (__bf16)k[3]};
                    const bf16x2 v01 = {(__bf16)v[0], (__bf16)v[1]};
                    const bf16x2 v23 = {(__bf16)v[2], (__bf16)v[3]};
                    wk[0] = __builtin_bit_cast(uint32_t, k01);
                    wk[1] = __builtin_bit_cast(uint32_t, k23);
                    wv[0] = __builtin_bit_cast(uint32_t, v01);
                    wv[1] = __builtin_bit_cast(uint32_t, v23);
                    *(u32x2*)(dK + d0) = wk;
                    *(u32x2*)(dV + d0) = wv;
                }
        }
    }
    if constexpr (FDQ) {
        // merge the four waves' dQ^T sums (fixed order) and write this
        // workgroup's partial: slot blockIdx.x of [BH][gridDim.x][M][D],
        // scaled by s. Register r of accumulator (j, db): d = 32 db +
        // 8 (r/4) + 4 hi + r%4, latent 32 j + l32.
        __syncthreads();  // staged rows and tiles are no longer read
        float* mbuf = (float*)bsm;
        constexpr int PER = MBX * DB * 16 * 64;
        if (wave > 0) {
            float* d0 = mbuf + (wave - 1) * PER;
#pragma unroll
            for (int j = 0; j < MBX; ++j)
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) d0[((j * DB + db) * 16 + r) * 64 + lane] = dq[j][db][r];
        }
        __syncthreads();
        if (wave == 0) {
            for (int t = 0; t < 3; ++t) {
                const float* s0 = mbuf + t * PER;
#pragma unroll
                for (int j = 0; j < MBX; ++j)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) dq[j][db][r] += s0[((j * DB + db) * 16 + r) * 64 + lane];
            }
#pragma unroll
            for (int j = 0; j < MBX; ++j) {
                const int m = 32 * j + l32;
                if (j < MB && m < M) {
                    float* dst = a.part + (((int64_t)bh * gridDim.x + blockIdx.x) * M + m) * D;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const f32x4 v = {a.s * dq[j][db][4 * g4], a.s * dq[j][db][4 * g4 + 1],
                                             a.s * dq[j][db][4 * g4 + 2], a.s * dq[j][db][4 * g4 + 3]};
                            *(f32x4*)(dst + 32 * db + 8 * g4 + 4 * hi) = v;
                        }
                }
            }
        }
    }
}

// Latent-side backward products, split over token chunks like the encode:
//   DQ = false: dZ[m]  = sum_n Bt[n][m] dY[n]
//   DQ = true:  dQ[m]  = s sum_n dl[m][n] K[n]
// Grid (chunks C, B*H); the 4 waves share the chunk's tokens and split the
// latent blocks (wave w owns blocks w, w + 4, ...). Per 32-token sub-block a
// wave loads the token rows straight into MFMA A operands in enc_row_token
// order (rows = tokens of S^T = K Q^T), so registers 8 kp .. 8 kp + 7 of a lane
// hold tokens 16 kp + 8 hi + 0..7: the k-slots of the accumulation's B
// operand. The accumulation's A operand (dY^T or K^T) comes from a transposed
// read of the same rows, which the wave also writes to its own LDS tile in
// natural order. Per-chunk partials go to a.part [BH][C][M][D].
// ENC (with DQ): the encode's backward alone, dl = A (dZ V^T - gam), for the
// first stage of the FLARE++ backward: no decode weights, no dY.
template <int D, bool DQ, int MBW, bool ENC = false>  // MBW: latent blocks per wave at most
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 && !DQ ? 2 : 1))) void bw_lat_bf16(
    BackwardArgs a) {
    constexpr int KB = D / 16, DB = D / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char bsm[];
    const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = blockIdx.x, bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = (M + 31) & ~31, MB = Mp / 32;
    const int n0 = chunk * a.chunk_len, n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    unsigned char* qs = bsm;
    unsigned char* zs = qs + Mp * 2 * D;                 // DQ only
    unsigned char* dzs = zs + (DQ ? Mp * 2 * D : 0);     // DQ only
    unsigned char* tt = dzs + (DQ ? Mp * 2 * D : 0) + wave * 32 * 2 * D;  // this wave's token rows
    stage_rows<D>(qs, (const uint16_t*)a.Q + (int64_t)h * M * D, M, Mp, tid, 256);
    if constexpr (DQ) {
        stage_rows<D>(zs, a.Z + (int64_t)bh * M * D, M, Mp, tid, 256);
        stage_rows<D>(dzs, a.dZ + (int64_t)bh * M * D, M, Mp, tid, 256);
    }
    __syncthreads();
    // NL latent groups of up to MBW blocks x TS token streams: the waves of a
    // group split the chunk's sub-blocks and merge at the end, so each token
    // row a wave loads serves up to MBW latent blocks
    const int NL = min(4, (MB + MBW - 1) / MBW), TS = 4 / NL;
    const int lg = wave % NL, ts = wave / NL;
    const int nmb = (ts < TS && MB > lg) ? (MB - lg + NL - 1) / NL : 0;  // this wave's latent blocks
    // per latent (lane column) of each owned block: lambda = mu* + log2 sig*
    // (+inf for padding) and gam
    float lam[MBW], gm[MBW];
    f32x16 acc[MBW][DB];
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
        const int m = 32 * (lg + NL * j) + l32;
        const int64_t r = (int64_t)bh * M + min(m, M - 1);
        lam[j] = (DQ && m < M) ? a.zmu[r] + __log2f(a.zsig[r]) : INFINITY;
        gm[j] = (DQ && m < M) ? a.gam[r] : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[j][db] = f32x16{};
    }
    const int64_t sn = a.sn;
    const uint16_t* Kb = (const uint16_t*)a.K + head_base(a, bh);
    const uint16_t* Vb = (const uint16_t*)a.V + head_base(a, bh);
    const uint16_t* Gb = (const uint16_t*)a.dY + head_base(a, bh);
    const float* nub = a.nu + (int64_t)bh * N;
    const float* delb = a.del + (int64_t)bh * N;
    const int prow = enc_row_token(l32);
    const int g = lane >> 4, gi = lane & 15;
    // This sub-block's token rows and per-token statistics (one token per
    // lane, spread to the register layout by lane permutes); the next
    // sub-block's are loaded while this one is processed (clamped to this
    // one at the chunk's end, so the loads are unconditional and the
    // compiler's wait before the first use covers exactly them). (Loading
    // each sub-block's rows at its start instead, which lets the D = 64 dZ
    // form run three waves per SIMD, measured 7% slower on MI355X.)
    bf16x8 kA[KB], gA[KB], vA[KB], kP[KB], gP[KB], vP[KB];
    float nuP = 0.0f, deP = 0.0f;
    auto load = [&](int t) {
        const int nv = n1 - t, tn = t + min(prow, nv - 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t o = tn * sn + 16 * kb + 8 * hi;
            kP[kb] = *(const bf16x8*)(Kb + o);
            if constexpr (!ENC) gP[kb] = *(const bf16x8*)(Gb + o);
            if constexpr (DQ) vP[kb] = *(const bf16x8*)(Vb + o);
        }
        if constexpr (!ENC) {
            const int tc = t + min(l32, nv - 1);
            nuP = nub[tc];
            if constexpr (DQ) deP = delb[tc];
        }
    };
    int t0 = n0 + 32 * ts;
    if (nmb > 0 && t0 < n1) load(t0);
    for (; nmb > 0 && t0 < n1; t0 += 32 * TS) {
        const int nv = n1 - t0;  // valid tokens in this sub-block (>= 1)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kA[kb] = kP[kb];
            gA[kb] = gP[kb];
            vA[kb] = vP[kb];
        }
        const float nuc = nuP, dec = deP;
        load(t0 + 32 * TS < n1 ? t0 + 32 * TS : t0);
        // the accumulation's source rows (K for dQ, dY for dZ) in natural
        // order into this wave's tile; rows past the chunk are zero, so their
        // (finite) weights add nothing
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            *(bf16x8*)(tt + tile_off<D>(prow, 2 * kb + hi)) = prow < nv ? (DQ ? kA[kb] : gA[kb]) : zero8();
        // per token (register i: token 16 (i/8) + 8 hi + i%8): nu' and -del
        // (past the chunk: the last token's, with zero rows above); the
        // Z dY^T products start from -del, so the matrix core leaves
        // dY.Z - del
        float nur[16];
        f32x16 nder;
        if constexpr (!ENC) {
            const float ndec = -dec;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tk = 16 * (i >> 3) + 8 * hi + (i & 7);
                nur[i] = __shfl(nuc, tk, 64);
                nder[i] = DQ ? __shfl(ndec, tk, 64) : 0.0f;
            }
        }
        // the transposed operands of this sub-block (same for every latent block)
        auto taddr = [&](int kp, int db, int second) {
            const int row = 16 * kp + 8 * (g >> 1) + (gi >> 2) + 4 * second;
            const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
            return tt + tile_off<D>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
        };
        bf16x8 tA[2][DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
            lds_tr_op2_c(taddr(0, db, 0), taddr(0, db, 1), taddr(1, db, 0), taddr(1, db, 1), tA[0][db],
                         tA[1][db]);
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            if (j >= nmb) break;
            const int mb = lg + NL * j;
            bf16x8 qB[KB], zB[KB], dzB[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = tile_off<D>(32 * mb + l32, 2 * kb + hi);
                qB[kb] = *(const bf16x8*)(qs + off);
                if constexpr (DQ) {
                    zB[kb] = *(const bf16x8*)(zs + off);
                    dzB[kb] = *(const bf16x8*)(dzs + off);
                }
            }
            f32x16 S = mfma(kA[0], qB[0], f32x16{});
#pragma unroll
            for (int kb = 1; kb < KB; ++kb) S = mfma(kA[kb], qB[kb], S);
            f32x16 GY, GV;
            if constexpr (DQ) {
                GV = mfma(vA[0], dzB[0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) GV = mfma(vA[kb], dzB[kb], GV);
                if constexpr (!ENC) {
                    GY = mfma(gA[0], zB[0], nder);
#pragma unroll
                    for (int kb = 1; kb < KB; ++kb) GY = mfma(gA[kb], zB[kb], GY);
                }
            }
            bf16x8 pw[2];
            // The decode weight of a padded latent (zero row) can overflow
            // where nu' < -128; no clamp is applied: its weights only reach
            // the padded latent's own output column, which is not stored.
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float w;
                if constexpr (ENC) {
                    w = exp2_fast(fmaf(S[i], c, -lam[j])) * (GV[i] - gm[j]);
                } else {
                    // decode weight Bt[n][m] (0 past the chunk)
                    const float p_d = exp2_fast(fmaf(S[i], c, -nur[i]));
                    w = p_d;
                    if constexpr (DQ) {
                        const float p_e = exp2_fast(fmaf(S[i], c, -lam[j]));
                        w = fmaf(p_d, GY[i], p_e * (GV[i] - gm[j]));
                    }
                }
                pw[i >> 3][i & 7] = (__bf16)w;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[j][db] = mfma(tA[0][db], pw[0], acc[j][db]);
                acc[j][db] = mfma(tA[1][db], pw[1], acc[j][db]);
            }
        }
    }
    if (TS > 1) {  // merge the token streams of each latent group (fixed order)
        __syncthreads();  // staged rows and tiles are no longer read
        float* mbuf = (float*)bsm;
        constexpr int PER = MBW * DB * 16 * 64;
        if (ts > 0) {
            float* d0 = mbuf + ((ts - 1) * NL + lg) * PER;
#pragma unroll
            for (int j = 0; j < MBW; ++j)
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) d0[((j * DB + db) * 16 + r) * 64 + lane] = acc[j][db][r];
        }
        __syncthreads();
        if (ts == 0) {
            for (int t = 1; t < TS; ++t) {
                const float* s0 = mbuf + ((t - 1) * NL + lg) * PER;
#pragma unroll
                for (int j = 0; j < MBW; ++j)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[j][db][r] += s0[((j * DB + db) * 16 + r) * 64 + lane];
            }
        }
    }
    // acc[j][db] register r: d = 32 db + 8 (r/4) + 4 hi + r%4, latent column l32
    const float scale = DQ ? a.s : 1.0f;
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
        if (ts != 0 || j >= nmb) break;
        const int m = 32 * (lg + NL * j) + l32;
        if (m < M) {
            float* dst = a.part + (((int64_t)bh * gridDim.x + chunk) * M + m) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 v = {scale * acc[j][db][4 * g4], scale * acc[j][db][4 * g4 + 1],
                                     scale * acc[j][db][4 * g4 + 2], scale * acc[j][db][4 * g4 + 3]};
                    *(f32x4*)(dst + 32 * db + 8 * g4 + 4 * hi) = v;
                }
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
        case 96: return FN<96>(a, s);    \
        case 128: return FN<128>(a, s);  \
        default: return hipErrorInvalidValue; \
    }

template <int D>
hipError_t stats_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid((a.N + kTokPerBlock - 1) / kTokPerBlock, a.BH);
    if (a.bf16)
        FLARE_LAUNCH((bw_stats<D, uint16_t>), grid, dim3(256), 0, s, a);
    else
        FLARE_LAUNCH((bw_stats<D, float>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t dz_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH, (a.M + 127) / 128);
    if (a.bf16)
        FLARE_LAUNCH((bw_latent<D, uint16_t, false>), grid, dim3(256), 0, s, a);
    else
        FLARE_LAUNCH((bw_latent<D, float, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t dq_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH, (a.M + 127) / 128);
    if (a.bf16)
        FLARE_LAUNCH((bw_latent<D, uint16_t, true>), grid, dim3(256), 0, s, a);
    else
        FLARE_LAUNCH((bw_latent<D, float, true>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
template <int D>
hipError_t dkdv_d(const BackwardArgs& a, hipStream_t s) {
    dim3 grid((a.N + kTokPerBlock - 1) / kTokPerBlock, a.BH);
    if (a.bf16)
        FLARE_LAUNCH((bw_dkdv<D, uint16_t>), grid, dim3(256), 0, s, a);
    else
        FLARE_LAUNCH((bw_dkdv<D, float>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool bw_bf16_fits(int M, int D) {
    // Q, Z and dZ of the head (and small per-latent or per-wave buffers) in
    // one CU's LDS; at D = 64 up to M = 256, at D = 128 up to M = 128
    const int Mp = (M + 31) / 32 * 32;
    return (D == 32 || (D == 64 && Mp <= 256) || (D == 128 && Mp <= 128)) &&
           3 * Mp * 2 * D + 4 * 32 * 2 * D + 12 * Mp <= 163840;
}

namespace {
// Workgroups per (b, h) of the token-side kernels: about 1024 in all, at most
// one per four 32-token blocks.
int tok_groups(const BackwardArgs& a, int nwv = 4) {
    const int nblk = (a.N + 31) / 32;
    return std::max(1, std::min((4096 / nwv + a.BH - 1) / a.BH, (nblk + nwv - 1) / nwv));
}
template <typename F>
hipError_t launch_bw_tok(F fn, const BackwardArgs& a, int lds, hipStream_t s, int G = 0, int nwv = 4) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    FLARE_LAUNCH(fn, dim3(G > 0 ? G : tok_groups(a, nwv), a.BH), dim3(64 * nwv), lds, s, a);
    return hipGetLastError();
}
}  // namespace

int bw_fused_dq_groups(const BackwardArgs& a) {
    const int Mp = (a.M + 31) / 32 * 32;
    // (D = 64: two latent blocks, whose sums fill the registers of the one
    // wave per SIMD the kernel runs at)
    if (!a.bf16 || a.enc_only || !((a.D == 32 && Mp <= 128) || (a.D == 64 && Mp <= 64)) || a.C < 1) return 0;
    return std::min(tok_groups(a), a.C);
}

int bw_fused_dz_groups(const BackwardArgs& a) {
    const int Mp = (a.M + 31) / 32 * 32;
    if (!a.bf16 || a.enc_only || !((a.D == 32 && Mp <= 128) || (a.D == 64 && Mp <= 64)) || a.C < 1) return 0;
    return std::min(tok_groups(a), a.C);
}

hipError_t launch_bw_stats_bf16(const BackwardArgs& a, hipStream_t s) {
    const int Mp = (a.M + 31) / 32 * 32, lds = 2 * Mp * 2 * a.D + 16;
    if (const int fg = bw_fused_dz_groups(a)) {
        // dZ fused in: per-wave dY and Bt tiles, and the four waves' sums
        // (64 registers each) merged through LDS at the end
        const int mbx = a.D == 64 ? 2 : 4;
        const int lds_f = std::max(lds + 4 * (32 * 2 * a.D + mbx * 32 * 64), 3 * 16 * 64 * 64 * 4 / 16);
        if (a.D == 32) return launch_bw_tok(bw_stats_bf16<32, true>, a, lds_f, s, fg);
        return launch_bw_tok(bw_stats_bf16<64, true>, a, lds_f, s, fg);
    }
    if (a.D == 32) return launch_bw_tok(bw_stats_bf16<32>, a, lds, s);
    if (a.D == 64) return launch_bw_tok(bw_stats_bf16<64>, a, lds, s);
    if (a.D == 128) return launch_bw_tok(bw_stats_bf16<128>, a, lds, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bw_lat_bf16(const BackwardArgs& a, bool dq, hipStream_t s) {
    const int Mp = (a.M + 31) / 32 * 32;
    // latent blocks per wave: 4 at D = 32 (one wave covers M = 128) and at
    // D = 64 with 256 latents (two latent groups of two token streams: each
    // token row a wave loads serves twice the latents; 12-15% faster latent
    // kernels on MI355X than four groups of two blocks), else 2
    const int mbw = (a.D == 32 || (a.D == 64 && Mp == 256)) ? 4 : 2;
    const int nl = std::min(4, (Mp / 32 + mbw - 1) / mbw), ts = 4 / nl;
    const int merge = (ts - 1) * nl * mbw * (a.D / 32) * 16 * 64 * 4;  // token-stream merge
    const int lds = std::max((dq ? 3 : 1) * Mp * 2 * a.D + 4 * 32 * 2 * a.D, merge);
    auto go = [&](auto fn) -> hipError_t {
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
        }
        FLARE_LAUNCH(fn, dim3(a.C, a.BH), dim3(256), lds, s, a);
        return hipGetLastError();
    };
    if (dq && a.enc_only) {
        if (a.D == 32) return go(bw_lat_bf16<32, true, 4, true>);
        if (a.D == 64 && Mp == 256) return go(bw_lat_bf16<64, true, 4, true>);
        if (a.D == 64 && Mp <= 256) return go(bw_lat_bf16<64, true, 2, true>);
        if (a.D == 128 && Mp <= 128) return go(bw_lat_bf16<128, true, 2, true>);
        return hipErrorInvalidValue;
    }
    if (a.D == 32) return dq ? go(bw_lat_bf16<32, true, 4>) : go(bw_lat_bf16<32, false, 4>);
    if (a.D == 64 && Mp == 256) return dq ? go(bw_lat_bf16<64, true, 4>) : go(bw_lat_bf16<64, false, 4>);
    if (a.D == 64 && Mp <= 256) return dq ? go(bw_lat_bf16<64, true, 2>) : go(bw_lat_bf16<64, false, 2>);
    if (a.D == 128 && Mp <= 128) return dq ? go(bw_lat_bf16<128, true, 2>) : go(bw_lat_bf16<128, false, 2>);
    return hipErrorInvalidValue;
}

hipError_t launch_bw_dkdv_bf16(const BackwardArgs& a, hipStream_t s) {
    const int Mp = (a.M + 31) / 32 * 32;
    const int lds = (a.enc_only ? 2 : 3) * Mp * 2 * a.D + 12 * Mp;  // rows, then lam, -gam and the logits' start
    if (a.enc_only) {
        if (a.D == 32) return launch_bw_tok(bw_dkdv_bf16<32, true>, a, lds, s);
        if (a.D == 64 && Mp > 128) return launch_bw_tok(bw_dkdv_bf16<64, true, false, 4, 8>, a, lds, s, 0, 8);
        if (a.D == 64) return launch_bw_tok(bw_dkdv_bf16<64, true>, a, lds, s);
        if (a.D == 128 && Mp <= 192) return launch_bw_tok(bw_dkdv_bf16<128, true>, a, lds, s);
        return hipErrorInvalidValue;
    }
    if (const int fg = bw_fused_dq_groups(a)) {
        // dQ fused in: per-wave K and dl tiles, and the four waves' sums
        // (mbx latent blocks) merged through LDS at the end
        const int mbx = a.D == 64 ? 2 : 4;
        const int lds_f = std::max(lds + 4 * (32 * 2 * a.D + 32 * 64), 3 * mbx * (a.D / 32) * 16 * 64 * 4);
        if (a.D == 32) return launch_bw_tok(bw_dkdv_bf16<32, false, true>, a, lds_f, s, fg);
        return launch_bw_tok(bw_dkdv_bf16<64, false, true, 2>, a, lds_f, s, fg);
    }
    if (a.D == 32) return launch_bw_tok(bw_dkdv_bf16<32>, a, lds, s);
    if (a.D == 64 && Mp > 128) return launch_bw_tok(bw_dkdv_bf16<64, false, false, 4, 8>, a, lds, s, 0, 8);
    if (a.D == 64) return launch_bw_tok(bw_dkdv_bf16<64>, a, lds, s);
    if (a.D == 128 && Mp <= 192) return launch_bw_tok(bw_dkdv_bf16<128>, a, lds, s);  // 146 KB of LDS at 192
    return hipErrorInvalidValue;
}

bool backward_supports(int D) {
    return D == 8 || D == 16 || D == 24 || D == 32 || D == 48 || D == 64 || D == 96 || D == 128;
}

hipError_t launch_bw_stats(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(stats_d, a, s) }
hipError_t launch_bw_dz(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(dz_d, a, s) }
hipError_t launch_bw_dq(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(dq_d, a, s) }
hipError_t launch_bw_dkdv(const BackwardArgs& a, hipStream_t s) { FLARE_BW_DISPATCH(dkdv_d, a, s) }

// Per token: merge two latent ranges' statistics, each a log2-sum nu_r of
// 2^(c l) over its latents and del_r = <dY, Y_r> with Y_r normalised over
// the range: nu = log2(2^nu_a + 2^nu_b), del = (2^nu_a del_a + 2^nu_b del_b)
// / 2^nu (exact log-sum-exp merge), into the first pair.
__global__ __launch_bounds__(256) void bw_stats_merge_kernel(float* __restrict__ nu, float* __restrict__ del,
                                                             const float* __restrict__ nu2,
                                                             const float* __restrict__ del2, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float a = nu[i], b = nu2[i], m = fmaxf(a, b);
        const float wa = exp2f(a - m), wb = exp2f(b - m), w = wa + wb;
        nu[i] = m + log2f(w);
        del[i] = (wa * del[i] + wb * del2[i]) / w;
    }
}

hipError_t launch_bw_stats_merge(float* nu, float* del, const float* nu2, const float* del2, int64_t n,
                                 hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<int64_t>(8192, (n + 255) / 256);
    FLARE_LAUNCH(bw_stats_merge_kernel, dim3(blocks), dim3(256), 0, s, nu, del, nu2, del2, n);
    return hipGetLastError();
}

hipError_t launch_bw_dz_combine(const BackwardArgs& a, hipStream_t s) {
    const int64_t n = (int64_t)a.BH * a.M;  // one wave each, four per workgroup
    FLARE_LAUNCH(bw_dz_combine, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bw_dq_combine(const BackwardArgs& a, hipStream_t s) {
    const int64_t n = (int64_t)a.H * a.M * a.D;  // 64 entries per workgroup
    if (a.bf16)
        FLARE_LAUNCH(bw_dq_combine<uint16_t>, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, a);
    else
        FLARE_LAUNCH(bw_dq_combine<float>, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace flare
