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

__device__ __forceinline__ void combine_store(const CombineArgs& a, int bh, int m, int d, float mx, float den,
                                              const f32x4c& z);

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
    combine_store(a, bh, m, d, mx, den, z);
}

// The combine's outputs for one entry: merged offset and sum (optional), then
// Z in fp32 or the operator dtype, or Q' = Q + Z.
__device__ __forceinline__ void combine_store(const CombineArgs& a, int bh, int m, int d, float mx, float den,
                                              const f32x4c& z) {
    const int D = a.D;
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
// fp32 encode partials: grid (C, BH, latent groups); L consecutive lanes per
// latent, each holding D/L of its columns (L = 1, 2 or 4: more lanes when
// there are few latents, so that short chunks still fill a wave). K/V tiles
// of 64 tokens go through LDS (16-byte loads); each latent keeps its exact
// running maximum, sum and accumulator (the scalars in all L lanes). The dot
// products run as four independent partial sums over the lane's columns,
// closed across the L lanes by xor shuffles (shorter dependency chains;
// every chunk is short, so the chains, not the loads, set the time).
// ---------------------------------------------------------------------------
typedef float f32x4f __attribute__((ext_vector_type(4)));

template <int DL, int L>
__device__ __forceinline__ float dot4(const float* q, const float* k) {
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int d = 0; d < DL; d += 4) {
        const f32x4f kv = *(const f32x4f*)(k + d);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = fmaf(q[d + i], kv[i], s[i]);
    }
    float r = (s[0] + s[1]) + (s[2] + s[3]);
#pragma unroll
    for (int o = 1; o < L; o <<= 1) r += __shfl_xor(r, o, 64);
    return r;
}

// Exact online softmax of one query row q (this lane's DL columns) against
// `rows` LDS rows of D floats: keys kr, values vr (both already offset to
// this lane's columns), scores c * <q, k>, folded into the running (offset
// mu, sum, accumulator). Rows go four at a time: their four scores first,
// then one rescale to the largest, then their terms in row order; a tail of
// fewer than four goes one at a time. Every rescale is by 2^(mu_old - mu_new),
// so the ratio acc / sum is the softmax whatever the grouping.
template <int D, int L>
__device__ __forceinline__ void online_softmax_rows(const float* q, const float* kr, const float* vr, int rows,
                                                    float c, float& mu, float& sum, float* acc) {
    constexpr int DL = D / L;
    auto rescale = [&](float xm) {
        if (xm > mu) {
            const float alpha = (mu == -INFINITY) ? 0.0f : exp2f(mu - xm);
            sum *= alpha;
#pragma unroll
            for (int d = 0; d < DL; ++d) acc[d] *= alpha;
            mu = xm;
        }
    };
    auto add = [&](float x, const float* v) {
        const float p = exp2f(x - mu);
        sum += p;
#pragma unroll
        for (int d = 0; d < DL; d += 4) {
            const f32x4f vv = *(const f32x4f*)(v + d);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[d + i] = fmaf(p, vv[i], acc[d + i]);
        }
    };
    int r = 0;
    for (; r + 4 <= rows; r += 4) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = dot4<DL, L>(q, kr + (r + j) * D) * c;
        rescale(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
#pragma unroll
        for (int j = 0; j < 4; ++j) add(x[j], vr + (r + j) * D);
    }
    for (; r < rows; ++r) {
        const float x = dot4<DL, L>(q, kr + r * D) * c;
        rescale(x);
        add(x, vr + r * D);
    }
}

template <int D, int L>
__global__ __launch_bounds__(256) void encode_partial_f32(EncodeArgs a) {
    constexpr int T = 64, DL = D / L;
    __shared__ __attribute__((aligned(16))) float kt[T * D], vt[T * D];
    const int tid = threadIdx.x, nth = blockDim.x, j = tid % L;
    const int chunk = a.heads_fast ? blockIdx.y : blockIdx.x, bh = a.heads_fast ? blockIdx.x : blockIdx.y;
    const int m = blockIdx.z * (nth / L) + tid / L;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M;
    const int n0 = chunk * a.chunk_len, n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    const float* Kb = (const float*)a.K + (int64_t)b * a.sb + (int64_t)h * a.sh;
    const float* Vb = (const float*)a.V + (int64_t)b * a.sb + (int64_t)h * a.sh;
    const float* Qb = (const float*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const bool active = m < M;  // the same for the L lanes of a latent
    float q[DL], acc[DL];
#pragma unroll
    for (int d = 0; d < DL; ++d) {
        q[d] = active ? Qb[(int64_t)m * D + j * DL + d] : 0.0f;
        acc[d] = 0.0f;
    }
    float mu = -INFINITY, sig = 0.0f;
    for (int t0 = n0; t0 < n1; t0 += T) {
        const int nt = min(T, n1 - t0);
        // token rows are D contiguous floats (D a multiple of 8, rows 16-byte aligned)
        for (int e = tid; e < nt * (D / 4); e += nth) {
            const int r = e / (D / 4), d = 4 * (e % (D / 4));
            const int64_t g = (int64_t)(t0 + r) * a.sn + d;
            *(f32x4f*)(kt + r * D + d) = *(const f32x4f*)(Kb + g);
            *(f32x4f*)(vt + r * D + d) = *(const f32x4f*)(Vb + g);
        }
        __syncthreads();
        if (active) online_softmax_rows<D, L>(q, kt + j * DL, vt + j * DL, nt, c, mu, sig, acc);
        __syncthreads();
    }
    if (active) {
        const int64_t r = ((int64_t)bh * a.C + chunk) * a.Mp + m;
        if (j == 0) {
            a.out.mu[r] = mu;
            a.out.sig[r] = sig;
        }
#pragma unroll
        for (int d = 0; d < DL; ++d) a.out.acc[r * D + j * DL + d] = acc[d];
    }
}

// ---------------------------------------------------------------------------
// fp32 decode: grid (token blocks of 256 / L, BH); L consecutive lanes per
// token, each holding D/L of its columns. Exact online softmax over the
// latents, which stream through LDS in tiles of LT (Q and Z rows, 16-byte
// loads); the lanes of a group read the same latent row at a time (LDS
// broadcast).
// ---------------------------------------------------------------------------
template <int D, int L>
__global__ __launch_bounds__(256) void decode_f32(DecodeArgs a) {
    constexpr int LT = D <= 32 ? 64 : 32, DL = D / L, TPB = 256 / L;
    __shared__ __attribute__((aligned(16))) float qs[LT * D], zs[LT * D];
    const int bh = blockIdx.y, tid = threadIdx.x, j = tid % L;
    const int n = blockIdx.x * TPB + tid / L;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M;
    const bool active = n < N;  // every thread stages the tiles; the same for the L lanes of a token
    const float c = a.c;
    const float* Qb = (const float*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const float* Zb = (const float*)a.Z + (int64_t)bh * M * D;
    const int64_t row = (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)(active ? n : 0) * a.sn + j * DL;
    const float* kr = (const float*)a.K + row;
    float k[DL], y[DL];
#pragma unroll
    for (int d = 0; d < DL; d += 4) {
        const f32x4f kv = active ? *(const f32x4f*)(kr + d) : f32x4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            k[d + i] = kv[i];
            y[d + i] = 0.0f;
        }
    }
    float nu = -INFINITY, tau = 0.0f;
    for (int m0 = 0; m0 < M; m0 += LT) {
        const int lt = min(LT, M - m0);
        __syncthreads();  // the previous tile has been read
        for (int e = tid; e < lt * (D / 4); e += 256) {
            const int64_t g = (int64_t)m0 * D + 4 * e;
            *(f32x4f*)(qs + 4 * e) = *(const f32x4f*)(Qb + g);
            *(f32x4f*)(zs + 4 * e) = *(const f32x4f*)(Zb + g);
        }
        __syncthreads();
        if (active) online_softmax_rows<D, L>(k, qs + j * DL, zs + j * DL, lt, c, nu, tau, y);
    }
    if (active) {
        float* yr = (float*)a.Y + row;
#pragma unroll
        for (int d = 0; d < DL; ++d) yr[d] = y[d] / tau;
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    size_t n16) {
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        dst[i] = src[i];
}

// Peak probes: fixed instruction streams of known size over the whole chip,
// for the measurement harness to time. Each lane writes one float (the
// chains' results) so that nothing is elided.
typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef float f32x16p __attribute__((ext_vector_type(16)));

// Four independent chains of v_mfma_f32_32x32x16_bf16 per wave.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8p a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1e-3f * (lane + i));
        b[i] = (__bf16)(1e-3f * (lane - i));
    }
    f32x16p c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    out[blockIdx.x * 256 + threadIdx.x] = c0[0] + c1[5] + c2[10] + c3[15];
}

// Sixteen independent chains x <- 2^(-x) of v_exp_f32 per lane (values stay
// in [0.5, 1]; the negation is an operand modifier).
__global__ __launch_bounds__(256) void probe_exp_kernel(float* __restrict__ out, int iters) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 0.5f + 0.03f * j + 1e-5f * threadIdx.x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) r += x[j];
    out[blockIdx.x * 256 + threadIdx.x] = r;
}

// Streaming read of n16 16-byte vectors (grid-stride): each lane sums what it
// read into one float of `out`, so the loads are not elided.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, float* __restrict__ out, size_t n16) {
    uint32_t acc = 0;
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[blockIdx.x * 256 + threadIdx.x] = (float)(acc & 0xffff);
}

// Row copies in 4-byte words: copy i moves rows x words words, row r of src
// at src + r * sp, of dst at dst + r * dp (pitches in words). blockIdx.y
// selects the copy.
struct WordCopy {
    uint32_t* dst;
    const uint32_t* src;
    int64_t rows, words, sp, dp;
};
struct WordCopies {
    WordCopy c[kMaxCopies];
};
__global__ __launch_bounds__(256) void copy_rows_kernel(WordCopies b) {
    const WordCopy c = b.c[blockIdx.y];
    const int64_t n = c.rows * c.words;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
        const int64_t r = e / c.words, w = e - r * c.words;
        c.dst[r * c.dp + w] = c.src[r * c.sp + w];
    }
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

template <int D, int L>
hipError_t enc_f32_l(const EncodeArgs& a, hipStream_t s) {
    const int nth = enc_threads_f32(a.M, D);
    const int per = nth / L;  // latents per workgroup
    dim3 grid(a.heads_fast ? a.BH : a.C, a.heads_fast ? a.C : a.BH, (a.M + per - 1) / per), block(nth);
    FLARE_LAUNCH((encode_partial_f32<D, L>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t enc_f32(const EncodeArgs& a, hipStream_t s) {
    switch (f32_lanes_enc(a.M, D)) {
        case 1: return enc_f32_l<D, 1>(a, s);
        case 2: if constexpr (D % 8 == 0) return enc_f32_l<D, 2>(a, s); break;
        case 4: if constexpr (D % 16 == 0) return enc_f32_l<D, 4>(a, s); break;
    }
    return hipErrorInvalidValue;
}

template <int D, int L>
hipError_t dec_f32_l(const DecodeArgs& a, hipStream_t s) {
    dim3 grid((a.N + 256 / L - 1) / (256 / L), a.BH), block(256);
    FLARE_LAUNCH((decode_f32<D, L>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t dec_f32(const DecodeArgs& a, hipStream_t s) {
    switch (f32_lanes_dec(int64_t(a.N) * a.BH, D)) {
        case 1: return dec_f32_l<D, 1>(a, s);
        case 2: if constexpr (D % 8 == 0) return dec_f32_l<D, 2>(a, s); break;
        case 4: if constexpr (D % 16 == 0) return dec_f32_l<D, 4>(a, s); break;
    }
    return hipErrorInvalidValue;
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

// Lanes per latent (encode) or per token (decode): the largest of 4, 2, 1
// that divides D into 4-column groups, when it is worth it. The encode
// spreads few latents over more lanes (at most 64 / M lanes each); the decode
// does so when the tokens of all heads fill less than about 4096 wavefronts.
static int f32_lanes_fit(int want, int D) {
    int l = want >= 4 ? 4 : want >= 2 ? 2 : 1;
    while (l > 1 && D % (4 * l) != 0) l /= 2;
    return l;
}
int f32_lanes_enc(int M, int D) { return f32_lanes_fit(M <= 16 ? 4 : M <= 32 ? 2 : 1, D); }
int f32_lanes_dec(int64_t tokens, int D) { return f32_lanes_fit(tokens <= (int64_t(1) << 18) ? 4 : 1, D); }
int enc_threads_f32(int M, int D) {
    const int t = M * f32_lanes_enc(M, D);
    return t >= 256 ? 256 : (t + 63) / 64 * 64;
}

hipError_t launch_encode_f32(const EncodeArgs& a, hipStream_t s) { FLARE_F32_DISPATCH(enc_f32, a, s) }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) { FLARE_F32_DISPATCH(dec_f32, a, s) }

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.D % 4 != 0) return hipErrorInvalidValue;
    dim3 grid((a.M * (a.D / 4) + 255) / 256, a.BH), block(256);
    // groups of 8 chunks when that covers them all (fewer registers), else 16
    // (measured on MI355X: 32-chunk groups, or four lanes per entry splitting
    // the chunks, are slower at 32 chunks)
    if (a.C <= 8)
        FLARE_LAUNCH(combine_kernel<8>, grid, block, 0, s, a);
    else
        FLARE_LAUNCH(combine_kernel<16>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s) {
    if (bytes % 16 != 0) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    FLARE_LAUNCH(fill_zero_kernel, dim3(elementwise_blocks((int64_t)n16)), dim3(256), 0, s, (u32x4*)dst, n16);
    return hipGetLastError();
}

hipError_t launch_copy_rows(const CopyRows* c, int n, hipStream_t s) {
    if (n < 0 || n > kMaxCopies) return hipErrorInvalidValue;
    WordCopies b{};
    int k = 0;
    int64_t most = 0;
    for (int i = 0; i < n; ++i) {
        const CopyRows& x = c[i];
        if (x.row_bytes % 4 || x.src_pitch % 4 || x.dst_pitch % 4 || uintptr_t(x.dst) % 4 || uintptr_t(x.src) % 4)
            return hipErrorInvalidValue;
        if (x.rows <= 0 || x.row_bytes <= 0) continue;
        b.c[k++] = {(uint32_t*)x.dst, (const uint32_t*)x.src, x.rows, x.row_bytes / 4, x.src_pitch / 4,
                    x.dst_pitch / 4};
        most = std::max(most, x.rows * (x.row_bytes / 4));
    }
    if (k == 0) return hipSuccess;
    FLARE_LAUNCH(copy_rows_kernel, dim3(elementwise_blocks(most), k), dim3(256), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_widen(const void* src, float* dst, int64_t n, bool bf16, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (bf16)
        FLARE_LAUNCH(widen_kernel<uint16_t>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (const uint16_t*)src, dst, n);
    else
        FLARE_LAUNCH(widen_kernel<float>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (const float*)src, dst, n);
    return hipGetLastError();
}

hipError_t launch_batch_sum(void* dst, const void* base, const void* add, int B, int64_t n, bool bf16, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (bf16)
        FLARE_LAUNCH(batch_sum_kernel<uint16_t>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (uint16_t*)dst,
                           (const uint16_t*)base, (const uint16_t*)add, B, n);
    else
        FLARE_LAUNCH(batch_sum_kernel<float>, dim3(elementwise_blocks(n)), dim3(256), 0, s, (float*)dst,
                           (const float*)base, (const float*)add, B, n);
    return hipGetLastError();
}

hipError_t launch_probe(int kind, int iters, float* out, hipStream_t s) {
    const dim3 grid(kProbeLanes / 256), block(256);
    if (kind == 0)
        FLARE_LAUNCH(probe_mfma_kernel, grid, block, 0, s, out, iters);
    else if (kind == 1)
        FLARE_LAUNCH(probe_exp_kernel, grid, block, 0, s, out, iters);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_read(const void* src, size_t bytes, float* out, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    FLARE_LAUNCH(read_kernel, dim3(kProbeLanes / 256), dim3(256), 0, s, (const u32x4*)src, out, n16);
    return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    FLARE_LAUNCH(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, n16);
    return hipGetLastError();
}

}  // namespace flare
