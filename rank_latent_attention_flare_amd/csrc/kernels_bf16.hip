// FLARE / FLARE++ forward kernels for gfx950 (MI355X), bf16 storage with
// fp32 accumulation.
//
//  encode_partial_bf16  split-N encode: each workgroup streams one chunk of
//                       tokens of one (b, h) through LDS and keeps, per latent,
//                       an online-softmax state (offset, sum, accumulator).
//  decode_bf16          per-token softmax over the latents with Q and Z held in
//                       LDS; streams K once and writes Y once.
//
// Operator (FLARE skill page, steps 2 and 4; FLARE arXiv abstract): with
// s = 1/sqrt(D) and logits l[m][n] = s <Q[m], K[n]>, the encode is
// Z[m] = softmax_n(l[m][.]) V and the decode is Y[n] = softmax_m(l[.][n]) Z.
// Both contractions run on v_mfma_f32_32x32x16_bf16. In its 32x32 result,
// lane l holds column l%32 and rows 8*(r/4) + 4*(l/32) + r%4 in register r;
// its A and B operands hold row/column l%32 and k = 8*(l/32) + 0..7.
//
// Exponentials are taken in base 2 on logits pre-multiplied by
// c = s * log2(e), which leaves every softmax unchanged.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <cstdio>
#include <cstdlib>

#include "launch.h"

namespace flare {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Largest per-tile probability sum the encode accepts against its running
// offset before it re-centres (2^32; keeps every fp32 sum far from overflow).
constexpr float kSumLimit = 4294967296.0f;
// Smallest per-token probability sum the decode accepts against its
// Cauchy-Schwarz offset before it recomputes that block with exact maxima.
constexpr float kTauFloor = 9.094947017729282e-13f;  // 2^-40

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max of a value over the lane pair (l, l^32), same result in both lanes.
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// Byte offset of 16-byte chunk `ch` of row `row` in an LDS tile of bf16 rows
// of width D. Chunks are XOR-swizzled per row so that the row-strided reads
// of the MFMA operands spread over the banks.
template <int D>
__device__ __forceinline__ int tile_off(int row, int ch) {
    constexpr int CH = D / 8;
    constexpr int ROWS_PER_256B = (256 / (2 * D)) > 0 ? (256 / (2 * D)) : 1;
    const int sw = (row / ROWS_PER_256B) & (CH - 1);
    return row * (2 * D) + ((ch ^ sw) << 4);
}

// Token (0..31) held by MFMA row r of the encode's S^T = K Q^T product. The
// order makes accumulator registers 8j..8j+7 of a lane hold 8 consecutive
// tokens, i.e. exactly the k-slots the P.V product needs as its B operand.
__device__ __forceinline__ int enc_row_token(int r) {
    const int grp = r >> 3, hi = (r >> 2) & 1, lo = r & 3;
    return ((grp >> 1) << 4) + (hi << 3) + ((grp & 1) << 2) + lo;
}

__device__ __forceinline__ bf16x8 zero8() {
    u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, z);
}

// Probabilities of one 32-token sub-block for one 32-latent block:
// p = 2^(S*c - mu) rounded to bf16, packed as the two k-halves of the P.V B
// operand, and the sum of the rounded values.
__device__ __forceinline__ void enc_probs(const f32x16& S, float mu, float c, bf16x8& p0, bf16x8& p1,
                                          float& tsum) {
    const float nm = -mu;
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float t = 0.0f;
    bf16x8 pp[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e0 = exp2_fast(fmaf(S[8 * kp + 2 * j], c, nm));
            const float e1 = exp2_fast(fmaf(S[8 * kp + 2 * j + 1], c, nm));
            const bf16x2 p2 = {(__bf16)e0, (__bf16)e1};
            t = __builtin_amdgcn_fdot2_f32_bf16(p2, one, t, false);
            pp[kp][2 * j] = p2[0];
            pp[kp][2 * j + 1] = p2[1];
        }
    }
    p0 = pp[0];
    p1 = pp[1];
    tsum = t;
}

// ---------------------------------------------------------------------------
// K1: split-N encode partials.
//
// Workgroup = WM x WT waves for one (b, h) and one chunk of tokens. Wave
// (wm, wt) owns latents [32*MBW*wm, 32*MBW*(wm+1)) and, in every tile, the
// sub-blocks wt*SB .. wt*SB+SB-1 of 32 tokens. Tiles of T = 64 tokens of K
// and V stream from HBM straight into a ring of NS LDS stages with
// global_load_lds_dwordx4 (no staging registers); NS-1 tiles are in flight
// while one is consumed, and each wave waits only for its own transfers of
// the tile it needs (explicit vmcnt) before the workgroup barrier. Per
// sub-block:
//   S^T[tok][m] = K[tok] . Q[m]          (MFMA; A = K rows from LDS, B = Q)
//   p = 2^(S*c - mu[m])                  (lane-local: lane holds latent l%32)
//   acc^T[d][m] += V^T[d][tok] p[tok][m] (MFMA; A = V^T via LDS transpose reads)
// The offset mu[m] only moves when a tile's probability sum leaves
// (0, kSumLimit], so the common path needs no per-tile maximum; the rescale
// by 2^(mu_old - mu_new) is exact algebra and leaves the final ratio
// unchanged. At the end the WT token waves of a latent group merge their
// states through LDS and one writes (mu, sum, acc) for the chunk.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding global load, including the prefetched tiles).
// LDS ordering is explicit: each wave waits for its own transfers first.
__device__ __forceinline__ void raw_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16 bytes from global memory into LDS at lds_wave_base + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void*)g, (void*)lds_wave_base, 16, 0, 0);
}

template <int D, int MBW, int WM, int WT>
struct EncShape {
    static constexpr int KB = D / 16, DB = D / 32, CH = D / 8, RB = 2 * D;
    static constexpr int NW = WM * WT;
    static constexpr int T = 64;
    static constexpr int SB = T / (32 * WT);
    static constexpr int SBYTES = 2 * T * RB;  // K tile then V tile
    static constexpr int NS = (65536 / SBYTES) < 3 ? 3 : ((65536 / SBYTES) > 8 ? 8 : (65536 / SBYTES));
    static constexpr int IPW = T * CH / (64 * NW);  // transfers per wave per tensor per tile
    static constexpr int MERGE_BYTES = (WT - 1) * WM * MBW * (16 * DB + 2) * 64 * 4;
    static constexpr int SMEM = NS * SBYTES > MERGE_BYTES ? NS * SBYTES : MERGE_BYTES;
    static_assert(SB >= 1 && SB * 32 * WT == T, "tile split");
    static_assert(IPW >= 1 && IPW * 64 * NW == T * CH, "tile transfer split");
};

template <int D, int MBW, int WM, int WT>
__global__ __launch_bounds__(64 * WM * WT) void encode_partial_bf16(EncodeArgs a) {
    using Sh = EncShape<D, MBW, WM, WT>;
    constexpr int KB = Sh::KB, DB = Sh::DB, CH = Sh::CH, RB = Sh::RB, NW = Sh::NW, T = Sh::T, SB = Sh::SB;
    constexpr int NS = Sh::NS, IPW = Sh::IPW, SBYTES = Sh::SBYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sh::SMEM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;
    const int wm = wave % WM, wt = wave / WM;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = a.Mp;
    const int n0 = chunk * a.chunk_len;
    const int n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + (int64_t)bh * N * D;
    const uint16_t* __restrict__ Vb = (const uint16_t*)a.V + (int64_t)bh * N * D;
    const uint16_t* __restrict__ Qb = (const uint16_t*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;

    // This wave's latent queries as MFMA B operands (column m, k = d).
    bf16x8 qop[MBW][KB];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int m = 32 * (wm * MBW + mb) + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            qop[mb][kb] = (m < M) ? *(const bf16x8*)(Qb + (int64_t)m * D + 16 * kb + 8 * hi) : zero8();
    }

    float mu[MBW], ps[MBW];
    f32x16 acc[MBW][DB];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        mu[mb] = -INFINITY;
        ps[mb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][db][r] = 0.0f;
    }

    // Tile j of the chunk -> LDS stage `stage`. Transfer (i, wave) fills LDS
    // bytes [(i*NW + wave)*1024, +1024) of each tensor's tile, 16 per lane;
    // the lane fetches the global chunk that the swizzle places there. Rows
    // past the chunk end fetch the last valid token (finite data; their
    // logits are masked).
    auto issue = [&](int tile, int stage) {
        const int t0 = n0 + tile * T;
        unsigned char* st = smem + stage * SBYTES;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            const int row = p / CH, pos = p % CH;
            const int ch = pos ^ ((tile_off<D>(row, 0) - row * RB) >> 4);
            const int n = min(t0 + row, n1 - 1);
            const int64_t g = (int64_t)n * D + ch * 8;
            dma16(Kb + g, st + (i * NW + wave) * 1024);
            dma16(Vb + g, st + T * RB + (i * NW + wave) * 1024);
        }
    };

    const int ntiles = (n1 - n0 + T - 1) / T;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        if (j < ntiles) issue(j, j);

    for (int it = 0; it < ntiles; ++it) {
        // tile `it` is complete once at most the transfers of the (up to NS-2)
        // later tiles issued so far are outstanding
        if (it + NS - 2 < ntiles)
            wait_vmcnt<(NS - 2) * 2 * IPW>();
        else
            wait_vmcnt<0>();
        raw_barrier();
        if (it + NS - 1 < ntiles) issue(it + NS - 1, (it + NS - 1) % NS);
        const unsigned char* kt = smem + (it % NS) * SBYTES;
        const unsigned char* vt = kt + T * RB;
        const int valid = n1 - (n0 + it * T);
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int sb = wt * SB + j;
            const int nv = valid - 32 * sb;  // valid tokens in this sub-block
            if (nv <= 0) break;
            // S^T for the 32 tokens x (32 * MBW) latents.
            bf16x8 ka[KB];
            const int krow = 32 * sb + enc_row_token(l32);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ka[kb] = *(const bf16x8*)(kt + tile_off<D>(krow, 2 * kb + hi));
            f32x16 S[MBW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) S[mb][r] = 0.0f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) S[mb] = mfma(ka[kb], qop[mb][kb], S[mb]);
            }
            if (nv < 32) {
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tok = 16 * (i >> 3) + 8 * hi + (i & 7);
                        if (tok >= nv) S[mb][i] = -INFINITY;
                    }
            }
            bf16x8 pb[MBW][2];
            float ts[MBW];
            bool bad = false;
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                enc_probs(S[mb], mu[mb], c, pb[mb][0], pb[mb][1], ts[mb]);
                bad |= !(ts[mb] <= kSumLimit);
            }
            if (wave_any(bad)) {
                // Re-centre on the exact running maximum (rare: first tile of a
                // chunk, or a jump of the maximum by more than ~28 in log2).
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[mb][i]);
                    const float mnew = fmaxf(mu[mb], pair_max(mx) * c);
                    const float alpha = (mu[mb] == -INFINITY) ? 0.0f : exp2_fast(mu[mb] - mnew);
                    ps[mb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[mb][db] *= alpha;
                    mu[mb] = mnew;
                    enc_probs(S[mb], mu[mb], c, pb[mb][0], pb[mb][1], ts[mb]);
                }
            }
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) ps[mb] += ts[mb];
            // acc^T += V^T P^T. A operand = V^T rows d, k = 16 tokens, read
            // transposed from the row-major tile: lane i of each 16-lane group
            // receives element i%4 of source lanes 4k + i/4.
            const int g = lane >> 4, gi = lane & 15;
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
                const int row1 = 32 * sb + 16 * kp + 8 * (g >> 1) + (gi >> 2);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
                    const int off1 = tile_off<D>(row1, dcol >> 3) + ((dcol >> 2) & 1) * 8;
                    const int off2 = tile_off<D>(row1 + 4, dcol >> 3) + ((dcol >> 2) & 1) * 8;
                    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off1));
                    const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + off2));
                    const u32x2 w1 = __builtin_bit_cast(u32x2, r1);
                    const u32x2 w2 = __builtin_bit_cast(u32x2, r2);
                    const u32x4 w = {w1[0], w1[1], w2[0], w2[1]};
                    const bf16x8 va = __builtin_bit_cast(bf16x8, w);
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) acc[mb][db] = mfma(va, pb[mb][kp], acc[mb][db]);
                }
            }
        }
    }

    // Merge the WT token waves of each latent group (tile buffers are free
    // once every wave is past its last read; all transfers were waited for).
    if constexpr (WT > 1) {
        __syncthreads();
        float* mf = (float*)smem;
        constexpr int PER_WAVE = MBW * (16 * DB + 2) * 64;
        if (wt > 0) {
            float* dst = mf + ((wt - 1) * WM + wm) * PER_WAVE;
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                float* d2 = dst + mb * (16 * DB + 2) * 64;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) d2[(16 * db + r) * 64 + lane] = acc[mb][db][r];
                d2[(16 * DB) * 64 + lane] = mu[mb];
                d2[(16 * DB + 1) * 64 + lane] = ps[mb];
            }
        }
        __syncthreads();
        if (wt == 0) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                float mx = mu[mb];
                for (int w = 1; w < WT; ++w) {
                    const float* s2 = mf + ((w - 1) * WM + wm) * PER_WAVE + mb * (16 * DB + 2) * 64;
                    mx = fmaxf(mx, s2[(16 * DB) * 64 + lane]);
                }
                const float a0 = (mu[mb] == -INFINITY) ? 0.0f : exp2_fast(mu[mb] - mx);
                ps[mb] *= a0;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[mb][db] *= a0;
                for (int w = 1; w < WT; ++w) {
                    const float* s2 = mf + ((w - 1) * WM + wm) * PER_WAVE + mb * (16 * DB + 2) * 64;
                    const float mw = s2[(16 * DB) * 64 + lane];
                    const float aw = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - mx);
                    ps[mb] += aw * s2[(16 * DB + 1) * 64 + lane];
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[mb][db][r] += aw * s2[(16 * db + r) * 64 + lane];
                }
                mu[mb] = mx;
            }
        }
    }

    if (wt == 0) {
        const int64_t pbase = ((int64_t)bh * gridDim.x + chunk) * Mp;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int m = 32 * (wm * MBW + mb) + l32;
            const float sig = pair_sum(ps[mb]);
            if (m < Mp) {
                if (hi == 0) {
                    a.out.mu[pbase + m] = mu[mb];
                    a.out.sig[pbase + m] = sig;
                }
                float* dst = a.out.acc + (pbase + m) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 v = {acc[mb][db][4 * g4], acc[mb][db][4 * g4 + 1], acc[mb][db][4 * g4 + 2],
                                         acc[mb][db][4 * g4 + 3]};
                        *(f32x4*)(dst + 32 * db + 8 * g4 + 4 * hi) = v;
                    }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K3: decode.
//
// Workgroup = kDecWaves waves for one (b, h); Q[h] (or Q'[b,h]) and Z[b,h] are
// staged once into LDS as bf16 (Z rounded to nearest-even from fp32 when it
// comes from the fused forward). Each wave then owns blocks of 32*TB tokens:
// it loads their K rows straight into MFMA B operands (next block in flight),
// and streams over the latents in blocks of 32:
//   S^T[m][tok] = Q[m] . K[tok]            (MFMA; A = Q from LDS)
//   p = 2^(S*c - nu[tok])                  (lane-local: lane holds token l%32)
//   Y^T[d][tok] += Z^T[d][m] p[m][tok]      (MFMA; A = Z^T from LDS)
// nu[tok] = c * max_m |Q[m]| * |K[tok]| bounds every logit of the token from
// above (Cauchy-Schwarz), so no maximum over the latents is needed and the
// registers do not grow with M. Softmax is invariant to the offset; if a
// token's probability sum falls below kTauFloor (offset too loose, rare) the
// block is recomputed with the exact per-token maximum. Y = (P Z) / sum(P),
// rounded to bf16 and stored as 32-byte runs per lane.
// ---------------------------------------------------------------------------
// Row d of the Z^T operand read by MFMA row q: makes output register r of
// lane l hold d = 16*(l/32) + r (contiguous 32 bytes of Y per lane).
__device__ __forceinline__ int dec_row_d(int q) { return 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3); }
// Position of latent m inside its 16-latent group in the Z^T LDS rows: lane
// half 0 needs latents {0-3, 8-11}, half 1 needs {4-7, 12-15}.
__device__ __forceinline__ int dec_zpos(int m) {
    const int r = m & 15;
    return (m & ~15) + (((r >> 2) & 1) << 3) + ((r >> 3) << 2) + (r & 3);
}

template <int D>
__host__ __device__ constexpr int dec_zt_stride(int Mp) {
    return 2 * Mp + 16;  // bytes per Z^T row (padded)
}

template <int D, typename ZT>
__global__ __launch_bounds__(64 * kDecWaves) void decode_bf16(DecodeArgs a) {
    constexpr int KB = D / 16, DB = D / 32, CH = D / 8, TB = kDecTB, NW = kDecWaves;
    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = a.Mp, Mb = Mp / 32;
    const float c = a.c;
    const int zs = dec_zt_stride<D>(Mp);
    unsigned char* qs = dsm;                  // [Mp][D] bf16, swizzled
    unsigned char* zt = dsm + Mp * 2 * D;     // [D][zs bytes]
    float* red = (float*)(zt + D * zs);       // [NW] reduction scratch
    const uint16_t* __restrict__ Qb = (const uint16_t*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const ZT* __restrict__ Zb = (const ZT*)a.Z + (int64_t)bh * M * D;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + (int64_t)bh * N * D;
    uint16_t* __restrict__ Yb = (uint16_t*)a.Y + (int64_t)bh * N * D;

    // ---- stage Q (bf16, swizzled rows) and Z^T (bf16, permuted latents)
    for (int p = tid; p < Mp * CH; p += 64 * NW) {
        const int m = p / CH, ch = p % CH;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < M) v = *(const u32x4*)(Qb + (int64_t)m * D + ch * 8);
        *(u32x4*)(qs + tile_off<D>(m, ch)) = v;
    }
    for (int e = tid; e < Mp * D; e += 64 * NW) {
        const int m = e / D, d = e % D;
        __bf16 z = (__bf16)0.0f;
        if (m < M) {
            if constexpr (sizeof(ZT) == 4)
                z = (__bf16)(float)Zb[(int64_t)m * D + d];
            else
                z = __builtin_bit_cast(__bf16, (uint16_t)Zb[(int64_t)m * D + d]);
        }
        *(__bf16*)(zt + d * zs + 2 * dec_zpos(m)) = z;
    }
    __syncthreads();
    // largest latent norm (for the per-token Cauchy-Schwarz offset)
    float qn2 = 0.0f;
    for (int m = tid; m < M; m += 64 * NW) {
        float s2 = 0.0f;
        for (int ch = 0; ch < CH; ++ch) {
            const bf16x8 v = *(const bf16x8*)(qs + tile_off<D>(m, ch));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f = (float)v[j];
                s2 = fmaf(f, f, s2);
            }
        }
        qn2 = fmaxf(qn2, s2);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qn2 = fmaxf(qn2, __shfl_xor(qn2, off, 64));
    if (lane == 0) red[wave] = qn2;
    __syncthreads();
    float qmax2 = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) qmax2 = fmaxf(qmax2, red[w]);
    const float cq = c * sqrtf(qmax2);

    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    const int nblk = (N + 32 * TB - 1) / (32 * TB);
    const int stride = gridDim.x * NW;
    int blk = blockIdx.x * NW + wave;

    bf16x8 kop[TB][KB], knx[TB][KB];
    auto kload = [&](int bk, bf16x8 (&dst)[TB][KB]) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int n = bk * 32 * TB + 32 * tb + l32;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                dst[tb][kb] = (bk < nblk && n < N) ? *(const bf16x8*)(Kb + (int64_t)n * D + 16 * kb + 8 * hi) : zero8();
        }
    };
    if (blk < nblk) kload(blk, kop);

    for (; blk < nblk; blk += stride) {
        kload(blk + stride, knx);  // next block in flight
        float nu[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            float s2 = 0.0f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x2 k2 = {kop[tb][kb][2 * j], kop[tb][kb][2 * j + 1]};
                    s2 = __builtin_amdgcn_fdot2_f32_bf16(k2, k2, s2, false);
                }
            nu[tb] = cq * sqrtf(pair_sum(s2));
        }

        f32x16 yac[TB][DB];
        float tau[TB];
        auto run = [&](const float (&off)[TB]) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                tau[tb] = 0.0f;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) yac[tb][db][r] = 0.0f;
            }
            for (int mb = 0; mb < Mb; ++mb) {
                bf16x8 qa[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    qa[kb] = *(const bf16x8*)(qs + tile_off<D>(32 * mb + l32, 2 * kb + hi));
                bf16x8 pb[TB][2];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    f32x16 S;
#pragma unroll
                    for (int r = 0; r < 16; ++r) S[r] = 0.0f;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) S = mfma(qa[kb], kop[tb][kb], S);
                    if (32 * mb + 32 > M) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int m = 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
                            if (m >= M) S[i] = -INFINITY;
                        }
                    }
                    const float nm = -off[tb];
                    float t = tau[tb];
#pragma unroll
                    for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float e0 = exp2_fast(fmaf(S[8 * kp + 2 * j], c, nm));
                            const float e1 = exp2_fast(fmaf(S[8 * kp + 2 * j + 1], c, nm));
                            const bf16x2 p2 = {(__bf16)e0, (__bf16)e1};
                            t = __builtin_amdgcn_fdot2_f32_bf16(p2, one, t, false);
                            pb[tb][kp][2 * j] = p2[0];
                            pb[tb][kp][2 * j + 1] = p2[1];
                        }
                    tau[tb] = t;
                }
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int d = 32 * db + dec_row_d(l32);
                        const bf16x8 za = *(const bf16x8*)(zt + d * zs + 2 * (32 * mb + 16 * kp + 8 * hi));
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) yac[tb][db] = mfma(za, pb[tb][kp], yac[tb][db]);
                    }
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) tau[tb] = pair_sum(tau[tb]);
        };
        run(nu);
        bool low = false;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) low |= !(tau[tb] >= kTauFloor);
        if (wave_any(low)) {
            // Exact per-token maxima over the latents, then recompute.
            float mx[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) mx[tb] = -INFINITY;
            for (int mb = 0; mb < Mb; ++mb) {
                bf16x8 qa[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    qa[kb] = *(const bf16x8*)(qs + tile_off<D>(32 * mb + l32, 2 * kb + hi));
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    f32x16 S;
#pragma unroll
                    for (int r = 0; r < 16; ++r) S[r] = 0.0f;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) S = mfma(qa[kb], kop[tb][kb], S);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int m = 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3);
                        if (m < M) mx[tb] = fmaxf(mx[tb], S[i]);
                    }
                }
            }
            float ex[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) ex[tb] = pair_max(mx[tb]) * c;
            run(ex);
        }
        // normalise, round, store
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int n = blk * 32 * TB + 32 * tb + l32;
            const float inv = 1.0f / tau[tb];
            if (n < N) {
                uint16_t* dst = Yb + (int64_t)n * D + 16 * hi;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    bf16x8 o0, o1;
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        o0[r] = (__bf16)(yac[tb][db][r] * inv);
                        o1[r] = (__bf16)(yac[tb][db][8 + r] * inv);
                    }
                    *(bf16x8*)(dst + 32 * db) = o0;
                    *(bf16x8*)(dst + 32 * db + 8) = o1;
                }
            }
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kop[tb][kb] = knx[tb][kb];
    }
}

template <int D, int MBW, int WM, int WT>
hipError_t launch_enc(const EncodeArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH), block(64 * WM * WT);
    hipLaunchKernelGGL((encode_partial_bf16<D, MBW, WM, WT>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_enc_d(const EncodeArgs& a, hipStream_t s) {
    const EncCfg cfg = enc_cfg_bf16(D, a.Mp / 32);
#define FLARE_ENC_CASE(MBW, WM, WT) \
    if (cfg.mbw == MBW && cfg.wm == WM && cfg.wt == WT) return launch_enc<D, MBW, WM, WT>(a, s);
    FLARE_ENC_CASE(1, 1, 2)
    FLARE_ENC_CASE(1, 2, 2)
    FLARE_ENC_CASE(1, 4, 1)
    if constexpr (D == 128) {
        FLARE_ENC_CASE(1, 8, 1)
    } else {
        FLARE_ENC_CASE(2, 4, 1)
        FLARE_ENC_CASE(2, 2, 1)
        FLARE_ENC_CASE(2, 2, 2)
        FLARE_ENC_CASE(2, 1, 2)
    }
#undef FLARE_ENC_CASE
    return hipErrorInvalidValue;
}

template <int D, typename ZT>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t s) {
    const int lds = dec_lds_bytes_bf16(a.Mp, D);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)decode_bf16<D, ZT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    dim3 grid(a.G, a.BH), block(64 * kDecWaves);
    hipLaunchKernelGGL((decode_bf16<D, ZT>), grid, block, lds, s, a);
    return hipGetLastError();
}

}  // namespace

EncCfg enc_cfg_bf16(int D, int Mb) {
    // Tuning override (tests and sweeps): "mbw,wm,wt"; must name an
    // instantiated shape that covers Mb latent blocks.
    if (const char* e = std::getenv("FLARE_TEST_ENC_CFG")) {
        int x = 0, y = 0, z = 0;
        if (std::sscanf(e, "%d,%d,%d", &x, &y, &z) == 3 && x * y >= Mb) return {x, y, z};
    }
    if (Mb <= 1) return {1, 1, 2};
    if (Mb <= 2) return {1, 2, 2};
    if (Mb <= 4) return {1, 4, 1};
    if (D == 128) return {1, 8, 1};
    return {2, 4, 1};
}

int enc_tile_tokens_bf16(EncCfg) { return 64; }
int enc_threads_bf16(EncCfg cfg) { return 64 * cfg.wm * cfg.wt; }

int dec_lds_bytes_bf16(int Mp, int D) { return Mp * 2 * D + D * (2 * Mp + 16) + 64; }

hipError_t launch_encode_bf16(const EncodeArgs& a, hipStream_t s) {
    switch (a.D) {
        case 32: return launch_enc_d<32>(a, s);
        case 64: return launch_enc_d<64>(a, s);
        case 128: return launch_enc_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
    switch (a.D) {
        case 32: return a.z_f32 ? launch_dec<32, float>(a, s) : launch_dec<32, uint16_t>(a, s);
        case 64: return a.z_f32 ? launch_dec<64, float>(a, s) : launch_dec<64, uint16_t>(a, s);
        case 128: return a.z_f32 ? launch_dec<128, float>(a, s) : launch_dec<128, uint16_t>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace flare
