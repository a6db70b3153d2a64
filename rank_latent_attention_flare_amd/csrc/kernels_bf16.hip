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
#include <algorithm>

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
// Smallest per-token probability sum the decode accepts against its offset
// before it recomputes that block with exact maxima. Above it the largest
// term is >= 2^-98 and every term within fp32 precision of it is a normal
// number, so a loose offset costs no accuracy.
constexpr float kTauFloor = 8.077935669463161e-28f;  // 2^-90
// Log2 of kSumLimit: an accepted encode tile has every probability <= 2^32,
// so c*S <= mu + 32 for every latent offset mu the encode reports.
constexpr float kSumLimitLog2 = 32.0f;

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
__device__ __forceinline__ bool wave_all(bool p) { return __ballot(!p) == 0; }

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

// Probabilities of one lane's 16 entries of a 32x32 block of logits S:
// p = 2^(c*S - off) (the scale applied in fp32, one fma per entry), rounded to
// bf16 and packed as the two k-halves (p0, p1) of an MFMA B operand.
__device__ __forceinline__ void exp2_pack(const f32x16& S, float c, float off, bf16x8& p0, bf16x8& p1) {
    const float nm = -off;
    bf16x8 pp[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pp[kp][j] = (__bf16)exp2_fast(fmaf(S[8 * kp + j], c, nm));
    }
    p0 = pp[0];
    p1 = pp[1];
}

// Column sums of a 32-column B operand pair on the matrix core.
//
// Read as the B operand of v_mfma_f32_16x16x32_bf16, the registers of a
// 32x32x16 B operand (lane l: column l%32, k-half l/32) put column
// n + 16*((l/16)&1) of the wide product into column n = l%16, k-group l/16, of
// the narrow one. With A[row][k-group g] = 1 where ((row/4)&1) == (g&1), else
// 0, output row r of column n sums both k-halves of wide column
// n + 16*((r/4)&1); the narrow result puts rows 4*(l/16)..+3 in lane l, so
// every register of lane l holds the sum of wide column l%32. Products with
// 1 and 0 are exact, so this is the fp32 sum of the bf16 values.
__device__ __forceinline__ bf16x8 colsum_selector(int lane) {
    const bool on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
    const uint32_t w = on ? 0x3f803f80u : 0u;
    const u32x4 v = {w, w, w, w};
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ f32x4 colsum(const bf16x8& sel, const bf16x8& p0, const bf16x8& p1, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p0, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p1, acc, 0, 0, 0);
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

// 16 bytes from global memory into LDS at lds_wave_base + 16 * lane. NT: the
// non-temporal cache policy (K and V are read once per pass).
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void*)g, (void*)lds_wave_base, 16, 0, NT ? 2 : 0);
}

// Transposed LDS reads (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 64-bit words of lanes 4k + i/4 of the group.
// Two reads form one 8 x bf16 MFMA operand; lds_tr_op2 reads two operands.
// It is inline asm that waits for its own results before returning: with the
// compiler builtin, the compiler drains every outstanding global->LDS
// transfer (vmcnt(0)) before the read, which would empty the prefetch ring on
// every sub-block. Callers order these reads after the transfers they need
// (explicit vmcnt wait, then barrier).
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
__device__ __forceinline__ void lds_tr_op2(const unsigned char* p1, const unsigned char* p2,
                                           const unsigned char* p3, const unsigned char* p4, bf16x8& o1,
                                           bf16x8& o2) {
    u32x2 w1, w2, w3, w4;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(w4)
        : "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3)), "v"(lds_addr(p4))
        : "memory");
    const u32x4 a = {w1[0], w1[1], w2[0], w2[1]};
    const u32x4 b = {w3[0], w3[1], w4[0], w4[1]};
    o1 = __builtin_bit_cast(bf16x8, a);
    o2 = __builtin_bit_cast(bf16x8, b);
}

template <int D, int MBW, int WM, int WT>
struct EncShape {
    static constexpr int KB = D / 16, DB = D / 32, CH = D / 8, RB = 2 * D;
    static constexpr int NW = WM * WT;
    static constexpr int T = 64;
    static constexpr int SB = T / (32 * WT);
    static constexpr int SBYTES = 2 * T * RB;  // K tile then V tile
    // ring depth: 4 stages of 8 KB tiles (D = 32; measured best on MI355X),
    // otherwise as many stages as fit in 64 KB, at least 3
    static constexpr int NS = SBYTES <= 8192 ? 4 : ((65536 / SBYTES) < 3 ? 3 : ((65536 / SBYTES) > 8 ? 8 : (65536 / SBYTES)));
    static constexpr int PIECES = T * CH / 64;     // 1 KB transfers per tensor per tile
    static constexpr int IPW = PIECES >= NW ? PIECES / NW : 1;  // per issuing wave
    static constexpr int NWI = PIECES / IPW;       // issuing waves: the first NWI
    static constexpr int MERGE_BYTES = (WT - 1) * WM * MBW * (16 * DB + 2) * 64 * 4;
    static constexpr int SMEM = NS * SBYTES > MERGE_BYTES ? NS * SBYTES : MERGE_BYTES;
    static_assert(SB >= 1 && SB * 32 * WT == T, "tile split");
    static_assert(IPW * NWI == PIECES && NWI <= NW, "tile transfer split");
};

template <int D, int MBW, int WM, int WT>
__global__ __launch_bounds__(64 * WM * WT) void encode_partial_bf16(EncodeArgs a) {
    using Sh = EncShape<D, MBW, WM, WT>;
    constexpr int KB = Sh::KB, DB = Sh::DB, CH = Sh::CH, RB = Sh::RB, NW = Sh::NW, T = Sh::T, SB = Sh::SB;
    constexpr int NS = Sh::NS, IPW = Sh::IPW, NWI = Sh::NWI, SBYTES = Sh::SBYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sh::SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    const int wm = wave % WM, wt = wave / WM;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = a.Mp;
    const int n0 = chunk * a.chunk_len;
    const int n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    const int64_t kvoff = (int64_t)b * a.sb + (int64_t)h * a.sh;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + kvoff;
    const uint16_t* __restrict__ Vb = (const uint16_t*)a.V + kvoff;
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

    // Per latent: offset mu (log2 units; -inf until the first re-centring),
    // sum of p (whole sum in both lanes of a latent) and accumulator.
    float mu[MBW], ps[MBW];
    f32x16 acc[MBW][DB];
    const bf16x8 csel = colsum_selector(lane);
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        mu[mb] = -INFINITY;
        ps[mb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][db][r] = 0.0f;
    }

    // Tile j of the chunk -> LDS stage `stage`. The first NWI waves move the
    // tile, IPW transfers per tensor each: transfer (i, wave) fills LDS bytes
    // [(i*NWI + wave)*1024, +1024) of each tensor's tile, 16 per lane; the
    // lane fetches the global chunk that the swizzle places there. Rows past
    // the chunk end fetch the last valid token (finite data; their logits are
    // masked). Waves that move nothing have no transfers to wait for.
    auto issue = [&](int tile, int stage) {
        if (wave >= NWI) return;
        const int t0 = n0 + tile * T;
        unsigned char* st = smem + stage * SBYTES;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int pc = i * NWI + wave;
            const int p = pc * 64 + lane;
            const int row = p / CH, pos = p % CH;
            const int ch = pos ^ ((tile_off<D>(row, 0) - row * RB) >> 4);
            const int n = min(t0 + row, n1 - 1);
            const int64_t g = (int64_t)n * a.sn + ch * 8;
            // V is read with the non-temporal policy: K, which the decode
            // reads again, then stays in the last-level caches when it fits
            // (measured 7-17% faster decodes on MI355X at 134 MB of K). K is
            // non-temporal too for the D = 64 shapes with two latent blocks
            // per wave (faster there; their K does not fit anyway).
            constexpr bool KNT = D >= 64 && MBW >= 2;
            dma16<KNT>(Kb + g, st + pc * 1024);
            dma16<true>(Vb + g, st + T * RB + pc * 1024);
        }
    };

    const int ntiles = (n1 - n0 + T - 1) / T;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        if (j < ntiles) issue(j, j);

    // Tile `it` (tail: the chunk's last, ragged tile, whose sub-blocks may be
    // partial or empty; full tiles carry no masking code).
    auto tile = [&](int it, bool tail) {
        const unsigned char* kt = smem + (it % NS) * SBYTES;
        const unsigned char* vt = kt + T * RB;
        const int valid = n1 - (n0 + it * T);
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int sb = wt * SB + j;
            const int nv = valid - 32 * sb;  // valid tokens in this sub-block
            if (tail && nv <= 0) break;
            // S^T for the 32 tokens x (32 * MBW) latents.
            bf16x8 ka[KB];
            const int krow = 32 * sb + enc_row_token(l32);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ka[kb] = *(const bf16x8*)(kt + tile_off<D>(krow, 2 * kb + hi));
            // V^T operands (A of acc^T += V^T P^T; k = 16 tokens), read
            // transposed from the row-major tile: lane i of each 16-lane group
            // receives element i%4 of source lanes 4k + i/4. Operand o covers
            // tokens 16*(o/DB).. and rows d = 32*(o%DB)..
            const int g = lane >> 4, gi = lane & 15;
            auto vaddr = [&](int kp, int db, int second) {
                const int row = 32 * sb + 16 * kp + 8 * (g >> 1) + (gi >> 2) + 4 * second;
                const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
                return vt + tile_off<D>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
            };
            constexpr int NOP = 2 * DB;
            bf16x8 va[NOP];
            auto read_v = [&]() {
#pragma unroll
                for (int o = 0; o < NOP; o += 2) {
                    const int kp0 = o / DB, db0 = o % DB, kp1 = (o + 1) / DB, db1 = (o + 1) % DB;
                    lds_tr_op2(vaddr(kp0, db0, 0), vaddr(kp0, db0, 1), vaddr(kp1, db1, 0), vaddr(kp1, db1, 1),
                               va[o], va[o + 1]);
                }
            };
            // At D >= 64 the reads are issued here, so their latency overlaps
            // the logits and the softmax (measured 3-4% faster on MI355X); at
            // D = 32 after the softmax (faster there).
            constexpr bool kVEarly = D >= 64;
            if constexpr (kVEarly) read_v();
            auto mask = [&](f32x16& X) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tok = 16 * (i >> 3) + 8 * hi + (i & 7);
                    if (tok >= nv) X[i] = -INFINITY;
                }
            };
            // logits S (bf16 products, fp32 accumulation)
            f32x16 S[MBW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                S[mb] = mfma(ka[0], qop[mb][0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) S[mb] = mfma(ka[kb], qop[mb][kb], S[mb]);
                if (tail) mask(S[mb]);
            }
            bf16x8 pb[MBW][2];
            float ts[MBW];
            bool bad = false;
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) exp2_pack(S[mb], c, mu[mb], pb[mb][0], pb[mb][1]);
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                ts[mb] = colsum(csel, pb[mb][0], pb[mb][1], f32x4{})[0];
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
                    exp2_pack(S[mb], c, mu[mb], pb[mb][0], pb[mb][1]);
                    ts[mb] = colsum(csel, pb[mb][0], pb[mb][1], f32x4{})[0];
                }
            }
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) ps[mb] += ts[mb];
            // acc^T += V^T P^T
            if constexpr (!kVEarly) read_v();
#pragma unroll
            for (int o = 0; o < NOP; ++o) {
                const int kp = o / DB, db = o % DB;
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) acc[mb][db] = mfma(va[o], pb[mb][kp], acc[mb][db]);
            }
        }
    };
    const bool ragged = (n1 - n0) % T != 0;
    const int nfull = ragged ? ntiles - 1 : ntiles;
    for (int it = 0; it < ntiles; ++it) {
        // tile `it` is complete once at most the transfers of the (up to NS-2)
        // later tiles issued so far are outstanding
        if (it + NS - 2 < ntiles)
            wait_vmcnt<(NS - 2) * 2 * IPW>();
        else
            wait_vmcnt<0>();
        raw_barrier();
        if (it + NS - 1 < ntiles) issue(it + NS - 1, (it + NS - 1) % NS);
        if (it == nfull) break;  // only the ragged tile is left
        tile(it, false);
    }
    if (ragged) tile(nfull, true);

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
            const float sig = ps[mb];
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
// K1, private-stream form (used when one wave's registers hold all latents).
//
// Workgroup = NWV waves for one (b, h) and one chunk. Every wave owns ALL
// latents and its own stream of 32-token sub-blocks (wave w takes sub-blocks
// w, w + NWV, ...), fed through a private ring of NSW LDS stages by
// global_load_lds. No workgroup barrier is needed until the final merge; the
// logit MFMAs of all latent blocks are issued before the softmax VALU work so
// the matrix core runs under it. Arithmetic is the same as the shared form.
// ---------------------------------------------------------------------------
template <int D, int MBW, int NWV>
struct EncPrivShape {
    static constexpr int KB = D / 16, DB = D / 32, CH = D / 8, RB = 2 * D;
    static constexpr int SBYTES = 2 * 32 * RB;  // K then V of one 32-token sub-block
    static constexpr int BUDGET = 65536;
    static constexpr int NSW0 = BUDGET / (NWV * SBYTES);
    static constexpr int NSW = NSW0 < 2 ? 2 : (NSW0 > 8 ? 8 : NSW0);
    static constexpr int IPS = 32 * CH / 64;  // transfers per tensor per stage
    static constexpr int MERGE_BYTES = NWV * MBW * (16 * DB + 2) * 65 * 4;
    static constexpr int RING = NWV * NSW * SBYTES;
    static constexpr int SMEM = RING > MERGE_BYTES ? RING : MERGE_BYTES;
    static_assert(IPS * 64 == 32 * CH, "stage transfer split");
};

template <int D, int MBW, int NWV>
__global__ __launch_bounds__(64 * NWV) void encode_partial_priv_bf16(EncodeArgs a) {
    using Sh = EncPrivShape<D, MBW, NWV>;
    constexpr int KB = Sh::KB, DB = Sh::DB, CH = Sh::CH, RB = Sh::RB, NSW = Sh::NSW, IPS = Sh::IPS;
    constexpr int SBYTES = Sh::SBYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sh::SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = a.Mp;
    const int n0 = chunk * a.chunk_len;
    const int n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    const int64_t kvoff = (int64_t)b * a.sb + (int64_t)h * a.sh;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + kvoff;
    const uint16_t* __restrict__ Vb = (const uint16_t*)a.V + kvoff;
    const uint16_t* __restrict__ Qb = (const uint16_t*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    unsigned char* ring = smem + wave * (NSW * SBYTES);

    bf16x8 qop[MBW][KB];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int m = 32 * mb + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            qop[mb][kb] = (m < M) ? *(const bf16x8*)(Qb + (int64_t)m * D + 16 * kb + 8 * hi) : zero8();
    }
    float mu[MBW], ps[MBW];  // ps: whole sum in both lanes of a latent
    f32x16 acc[MBW][DB];
    const bf16x8 csel = colsum_selector(lane);
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        mu[mb] = -INFINITY;
        ps[mb] = 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][db][r] = 0.0f;
    }

    const int nsb = (n1 - n0 + 31) / 32;                        // sub-blocks in the chunk
    const int nsub = nsb > wave ? (nsb - wave + NWV - 1) / NWV : 0;  // this wave's share
    // Byte offset of this lane's IPS 16-byte pieces inside a 32-token block
    // (row-major source, swizzled destination): the same for every block.
    const uint32_t rsb = (uint32_t)(2 * a.sn);  // bytes between token rows in HBM
    uint32_t loff[IPS];
    int lrow[IPS];
#pragma unroll
    for (int i = 0; i < IPS; ++i) {
        const int p = i * 64 + lane;
        const int row = p / CH, pos = p % CH;
        const int ch = pos ^ ((tile_off<D>(row, 0) - row * RB) >> 4);
        lrow[i] = row;
        loff[i] = (uint32_t)(row * rsb + ch * 16);
    }
    auto issue = [&](int k) {
        const int t0 = n0 + 32 * (wave + k * NWV);
        unsigned char* st = ring + (k % NSW) * SBYTES;
        const unsigned char* kb0 = (const unsigned char*)(Kb + (int64_t)t0 * a.sn);
        const unsigned char* vb0 = (const unsigned char*)(Vb + (int64_t)t0 * a.sn);
        if (t0 + 32 <= n1) {
#pragma unroll
            for (int i = 0; i < IPS; ++i) {
                dma16(kb0 + loff[i], st + i * 1024);
                dma16<true>(vb0 + loff[i], st + 32 * RB + i * 1024);
            }
        } else {  // ragged tail: rows past the chunk end repeat its last token
#pragma unroll
            for (int i = 0; i < IPS; ++i) {
                const uint32_t o = loff[i] - (uint32_t)max(0, t0 + lrow[i] - (n1 - 1)) * rsb;
                dma16(kb0 + o, st + i * 1024);
                dma16<true>(vb0 + o, st + 32 * RB + i * 1024);
            }
        }
    };
#pragma unroll
    for (int k = 0; k < NSW - 1; ++k)
        if (k < nsub) issue(k);

    // One 32-token sub-block k of this wave (tail: the chunk's last, ragged one).
    auto sub_block = [&](int k, bool tail) {
        const unsigned char* kt = ring + (k % NSW) * SBYTES;
        const unsigned char* vt = kt + 32 * RB;
        const int nv = n1 - (n0 + 32 * (wave + k * NWV));
        bf16x8 ka[KB];
        const int krow = enc_row_token(l32);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) ka[kb] = *(const bf16x8*)(kt + tile_off<D>(krow, 2 * kb + hi));
        // V^T operands of this sub-block (shared by every latent block)
        bf16x8 va[2][DB];
        const int g = lane >> 4, gi = lane & 15;
        auto vaddr = [&](int kp, int db, int second) {
            const int row = 16 * kp + 8 * (g >> 1) + (gi >> 2) + 4 * second;
            const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
            return vt + tile_off<D>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
        };
#pragma unroll
        for (int o = 0; o < 2 * DB; o += 2) {
            const int kp0 = o / DB, db0 = o % DB, kp1 = (o + 1) / DB, db1 = (o + 1) % DB;
            lds_tr_op2(vaddr(kp0, db0, 0), vaddr(kp0, db0, 1), vaddr(kp1, db1, 0), vaddr(kp1, db1, 1),
                       va[kp0][db0], va[kp1][db1]);
        }
        // latent blocks in turn; block mb+1's logits are in flight on the
        // matrix core while block mb's softmax runs on the VALU
        // logits of latent block mb against this sub-block (masked on the
        // ragged tail)
        auto logits = [&](int mb) {
            f32x16 S = mfma(ka[0], qop[mb][0], f32x16{});
#pragma unroll
            for (int kb = 1; kb < KB; ++kb) S = mfma(ka[kb], qop[mb][kb], S);
            if (tail) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int tok = 16 * (i >> 3) + 8 * hi + (i & 7);
                    if (tok >= nv) S[i] = -INFINITY;
                }
            }
            return S;
        };
        f32x16 Snext = logits(0);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            f32x16 S = Snext;
            if (mb + 1 < MBW) Snext = logits(mb + 1);
            bf16x8 p0, p1;
            exp2_pack(S, c, mu[mb], p0, p1);
            float ts = colsum(csel, p0, p1, f32x4{})[0];
            if (wave_any(!(ts <= kSumLimit))) {
                // re-centre this latent block on its exact running maximum
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[i]);
                const float mnew = fmaxf(mu[mb], pair_max(mx) * c);
                const float alpha = (mu[mb] == -INFINITY) ? 0.0f : exp2_fast(mu[mb] - mnew);
                ps[mb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[mb][db] *= alpha;
                mu[mb] = mnew;
                exp2_pack(S, c, mu[mb], p0, p1);
                ts = colsum(csel, p0, p1, f32x4{})[0];
            }
            ps[mb] += ts;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc[mb][db] = mfma(va[0][db], p0, acc[mb][db]);
                acc[mb][db] = mfma(va[1][db], p1, acc[mb][db]);
            }
        }
    };
    // The chunk's last sub-block may be ragged; it is always this wave's last.
    const bool ragged = nsub > 0 && n1 - (n0 + 32 * (wave + (nsub - 1) * NWV)) < 32;
    const int nfull = ragged ? nsub - 1 : nsub;
    for (int k = 0; k < nsub; ++k) {
        if (k + NSW - 2 < nsub)
            wait_vmcnt<(NSW - 2) * 2 * IPS>();
        else
            wait_vmcnt<0>();
        if (k + NSW - 1 < nsub) {
            // the stage refilled here was read in the previous iteration
            __builtin_amdgcn_s_waitcnt((0x3F & 15) | ((0x3F >> 4) << 14) | (7 << 4) | (0 << 8));
            issue(k + NSW - 1);
        }
        if (k == nfull) break;  // only the ragged sub-block is left (its data has landed)
        sub_block(k, false);
    }
    if (ragged) sub_block(nfull, true);

    // Merge the NWV waves' states (each saw a disjoint set of sub-blocks):
    // every wave parks its state in LDS in its register layout (rows of 65
    // floats, one per lane plus a pad against bank conflicts), then all threads
    // combine disjoint (latent, column) entries and write the chunk's partials.
    // Entry (m, d) of wave w sits at lane (m % 32) + 32 * ((d / 4) % 2),
    // register 4 * ((d % 32) / 8) + d % 4 of accumulator (m / 32, d / 32).
    __syncthreads();
    float* mf = (float*)smem;
    constexpr int RL = 65;
    constexpr int PER_WAVE = MBW * (16 * DB + 2) * RL;
    {
        float* dst = mf + wave * PER_WAVE;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[((mb * DB + db) * 16 + r) * RL + lane] = acc[mb][db][r];
            dst[(MBW * DB * 16 + 2 * mb) * RL + lane] = mu[mb];
            dst[(MBW * DB * 16 + 2 * mb + 1) * RL + lane] = ps[mb];
        }
    }
    __syncthreads();
    const int64_t pbase = ((int64_t)bh * gridDim.x + chunk) * Mp;
    const int mlim = min(Mp, 32 * MBW);
    for (int e = tid; e < mlim * D; e += 64 * NWV) {
        const int m = e / D, d = e - m * D;
        const int mb = m >> 5, l = m & 31, db = d >> 5, dd = d & 31;
        const int r = 4 * (dd >> 3) + (dd & 3), ln = l + 32 * ((dd >> 2) & 1);
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; ++w) mx = fmaxf(mx, mf[w * PER_WAVE + (MBW * DB * 16 + 2 * mb) * RL + l]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            const float* src = mf + w * PER_WAVE;
            const float mw = src[(MBW * DB * 16 + 2 * mb) * RL + l];
            const float aw = (mw == -INFINITY) ? 0.0f : exp2_fast(mw - mx);
            num = fmaf(aw, src[((mb * DB + db) * 16 + r) * RL + ln], num);
            den = fmaf(aw, src[(MBW * DB * 16 + 2 * mb + 1) * RL + l], den);
        }
        a.out.acc[(pbase + m) * D + d] = num;
        if (d == 0) {
            a.out.mu[pbase + m] = mx;
            a.out.sig[pbase + m] = den;
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
// The offset nu bounds every logit of the token from above, so no maximum over
// the latents is needed and the registers do not grow with M: after the fused
// encode, one nu per (b, h) = max_m mu*[m] + 32 from the encode's merged
// offsets; standalone, nu[tok] = c * max_m |Q[m]| * |K[tok]| (Cauchy-Schwarz).
// Softmax is invariant to the offset; if a token's probability sum falls below
// kTauFloor (offset too loose, rare) the block is recomputed with the exact
// per-token maximum. Y = (P Z) / sum(P),
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

// LONG: M > 256 (more than one group of 8 latent blocks; the group loop costs
// registers, so the common M <= 256 kernel is built without it).
template <int D, int TB, typename ZT, bool LONG>
__global__ __launch_bounds__(64 * kDecWaves) void decode_bf16(DecodeArgs a) {
    constexpr int KB = D / 16, DB = D / 32, CH = D / 8, NW = kDecWaves;
    const int Mp = a.Mp, MB = Mp / 32;
    const int zs = 2 * Mp + 16;  // bytes per Z^T row (padded)
    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M;
    const float c = a.c;
    unsigned char* qs = dsm;                  // [Mp][D] bf16, swizzled
    unsigned char* zt = dsm + Mp * 2 * D;     // [D][zs bytes]
    float* red = (float*)(zt + D * zs);       // [NW] reduction scratch
    const uint16_t* __restrict__ Qb = (const uint16_t*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const ZT* __restrict__ Zb = (const ZT*)a.Z + (int64_t)bh * M * D;
    const int64_t sn = a.sn;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + (int64_t)b * a.sb + (int64_t)h * a.sh;
    uint16_t* __restrict__ Yb = (uint16_t*)a.Y + (int64_t)b * a.sb + (int64_t)h * a.sh;

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
    // Offsets. With the encode's merged offsets mu*[m] (log2 units), every
    // logit of this (b, h) satisfies c*S <= max_m mu*[m] + 32, one offset for
    // all tokens. Without them, per token: c * max_m |Q[m]| * |K[tok]|
    // (Cauchy-Schwarz); here only max_m |Q[m]|^2 is prepared.
    const bool goff = a.zmu != nullptr;
    float red_in = goff ? -INFINITY : 0.0f;
    if (goff) {
        for (int m = tid; m < M; m += 64 * NW) red_in = fmaxf(red_in, a.zmu[(int64_t)bh * M + m]);
    } else {
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
            red_in = fmaxf(red_in, s2);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) red_in = fmaxf(red_in, __shfl_xor(red_in, off, 64));
    if (lane == 0) red[wave] = red_in;
    __syncthreads();
    float rmax = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) rmax = fmaxf(rmax, red[w]);
    const float cq = goff ? 0.0f : c * sqrtf(rmax);
    const float gnu = goff ? rmax + kSumLimitLog2 : 0.0f;

    const bf16x8 csel = colsum_selector(lane);
    const f32x16 zero16 = {};
    const int nblk = (N + 32 * TB - 1) / (32 * TB);
    const int stride = gridDim.x * NW;

    auto kload = [&](int bk, bf16x8 (&dst)[TB][KB]) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int n = bk * 32 * TB + 32 * tb + l32;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                dst[tb][kb] = (bk < nblk && n < N) ? *(const bf16x8*)(Kb + (int64_t)n * sn + 16 * kb + 8 * hi) : zero8();
        }
    };
    auto qread = [&](int mb, bf16x8 (&qa)[KB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qa[kb] = *(const bf16x8*)(qs + tile_off<D>(32 * mb + l32, 2 * kb + hi));
    };
    // softmax numerator and denominator of one 32-token block against the
    // latents of block mb, with per-token offsets off[]
    auto mask_tail = [&](int mb, f32x16& S) {
        // Rows m >= M. The limit passes through an empty asm statement so the
        // compares are made here, on the tail block only, instead of being
        // hoisted out of the token loop for every latent block.
        int lim = M - 32 * mb - 4 * hi;
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (8 * (i >> 2) + (i & 3) >= lim) S[i] = -INFINITY;
    };

    // One 64-token block: Y^T[d][tok] = sum_m Z^T[d][m] 2^(c S - nu)  and
    // tau[tok] = sum_m 2^(c S - nu), latents streamed in blocks of 32.
    auto process = [&](int bk, const bf16x8 (&kop)[TB][KB]) {
        float nu[TB];
        if (goff) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) nu[tb] = gnu;
        } else {
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
                nu[tb] = cq * __builtin_sqrtf(pair_sum(s2));
            }
        }
        f32x16 yac[TB][DB];
        float tau[TB];  // whole sum over the latents, both lanes of a token
        f32x4 tacc[TB];
        auto run = [&](const float (&off)[TB]) {
            // logits S = Q K of latent block qa against token block tb
            auto logit = [&](const bf16x8 (&qa)[KB], int tb) {
                f32x16 S = mfma(qa[0], kop[tb][0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) S = mfma(qa[kb], kop[tb][kb], S);
                return S;
            };
            // Full latent blocks first (logits of block mb in SS[mb % 2]), then
            // the padded block when M % 32 != 0, with its own logits.
            const int MBF = M >> 5;
            bf16x8 qa[KB];
            f32x16 SS[2][TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) tacc[tb] = f32x4{};
            if (MBF > 0) {
                qread(0, qa);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) SS[0][tb] = logit(qa, tb);
            }
            // One latent block whose logits are in S: the Z^T operands are
            // requested from LDS (and, with `next`, the next block's logits go
            // to the matrix core, into Sn) before the softmax runs on the VALU.
            auto mstep = [&](int mb, bool first, bool next, f32x16 (&S)[TB], f32x16 (&Sn)[TB]) {
                if (next) {
                    qread(mb + 1, qa);
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) Sn[tb] = logit(qa, tb);
                }
                bf16x8 za[2][DB];
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int d = 32 * db + dec_row_d(l32);
                        za[kp][db] = *(const bf16x8*)(zt + d * zs + 2 * (32 * mb + 16 * kp + 8 * hi));
                    }
                bf16x8 pb[TB][2];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    exp2_pack(S[tb], c, off[tb], pb[tb][0], pb[tb][1]);
                    tacc[tb] = colsum(csel, pb[tb][0], pb[tb][1], tacc[tb]);
                }
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb)
                            yac[tb][db] = mfma(za[kp][db], pb[tb][kp], (first && kp == 0) ? zero16 : yac[tb][db]);
            };
            // all full latent blocks in groups of 8,
            // each group unrolled: the two logit buffers alternate without
            // register copies (8 is even, so block mb's logits are always in
            // SS[mb % 2]); the first group is separate so that its first
            // block starts the accumulators from the zero constant
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j >= MBF) break;
                mstep(j, j == 0, j + 1 < MBF, SS[j & 1], SS[(j + 1) & 1]);
            }
            if constexpr (LONG) {
#pragma unroll 1
                for (int g = 8; g < MBF; g += 8) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (g + j >= MBF) break;
                        mstep(g + j, false, g + j + 1 < MBF, SS[j & 1], SS[(j + 1) & 1]);
                    }
                }
            }
            if (M & 31) {
                qread(MBF, qa);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    SS[0][tb] = logit(qa, tb);
                    mask_tail(MBF, SS[0][tb]);
                }
                if (MBF == 0)
                    mstep(0, true, false, SS[0], SS[1]);
                else
                    mstep(MBF, false, false, SS[0], SS[1]);
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) tau[tb] = tacc[tb][0];
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
#pragma unroll 1
            for (int mb = 0; mb < MB; ++mb) {
                bf16x8 qa[KB];
                qread(mb, qa);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    f32x16 S = zero16;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) S = mfma(qa[kb], kop[tb][kb], S);
                    if (32 * mb + 32 > M) mask_tail(mb, S);
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx[tb] = fmaxf(mx[tb], S[i]);
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
            const int n = bk * 32 * TB + 32 * tb + l32;
            const float inv = __builtin_amdgcn_rcpf(tau[tb]);
            if (n < N) {
                uint16_t* dst = Yb + (int64_t)n * sn + 16 * hi;
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
    };

    // Blocks blk, blk + stride, ... of this wave. K register sets in turn so
    // that the rows of the next block (D = 32) or the next two blocks (D >= 64,
    // measured faster there; at D = 32 the extra registers cost more) are
    // always in flight.
    int blk = blockIdx.x * NW + wave;
    if constexpr (D >= 64) {
        bf16x8 kA[TB][KB], kB[TB][KB], kC[TB][KB];
        kload(blk, kA);
        kload(blk + stride, kB);
        while (blk < nblk) {
            kload(blk + 2 * stride, kC);
            process(blk, kA);
            blk += stride;
            if (blk >= nblk) break;
            kload(blk + 2 * stride, kA);
            process(blk, kB);
            blk += stride;
            if (blk >= nblk) break;
            kload(blk + 2 * stride, kB);
            process(blk, kC);
            blk += stride;
        }
    } else {
        bf16x8 kA[TB][KB], kB[TB][KB];
        kload(blk, kA);
        while (blk < nblk) {
            kload(blk + stride, kB);
            process(blk, kA);
            blk += stride;
            if (blk >= nblk) break;
            kload(blk + stride, kA);
            process(blk, kB);
            blk += stride;
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
// Z[m]>. Two sweeps over the latents: the exact maximum, then the sums.
template <int D>
__global__ __launch_bounds__(256) void bw_stats_bf16(BackwardArgs a) {
    constexpr int KB = D / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char bsm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = (M + 31) & ~31, MB = Mp / 32;
    const float c = a.c;
    unsigned char* qs = bsm;
    unsigned char* zs = bsm + Mp * 2 * D;
    stage_rows<D>(qs, (const uint16_t*)a.Q + (int64_t)h * M * D, M, Mp, tid, 256);
    stage_rows<D>(zs, a.Z + (int64_t)bh * M * D, M, Mp, tid, 256);
    __syncthreads();
    const uint16_t* Kb = (const uint16_t*)a.K + (int64_t)bh * N * D;
    const uint16_t* Gb = (const uint16_t*)a.dY + (int64_t)bh * N * D;
    const int nblk = (N + 31) / 32;
    for (int blk = blockIdx.x * 4 + wave; blk < nblk; blk += gridDim.x * 4) {
        const int n = blk * 32 + l32, nn = min(n, N - 1);
        bf16x8 kop[KB], gop[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            kop[kb] = *(const bf16x8*)(Kb + (int64_t)nn * D + 16 * kb + 8 * hi);
            gop[kb] = *(const bf16x8*)(Gb + (int64_t)nn * D + 16 * kb + 8 * hi);
        }
        auto rows = [&](const unsigned char* t, int mb, bf16x8 (&op)[KB]) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) op[kb] = *(const bf16x8*)(t + tile_off<D>(32 * mb + l32, 2 * kb + hi));
        };
        // register i holds latent 32 mb + 8 (i/4) + 4 hi + i%4 (natural rows)
        auto valid = [&](int mb, int i) { return 32 * mb + 8 * (i >> 2) + 4 * hi + (i & 3) < M; };
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
        const float nu = pair_max(mx) * c;
        float tau = 0.0f, pg = 0.0f;
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
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = valid(mb, i) ? exp2_fast(fmaf(S[i], c, -nu)) : 0.0f;
                tau += p;
                pg = fmaf(p, G[i], pg);
            }
        }
        tau = pair_sum(tau);
        pg = pair_sum(pg);
        if (n < N && hi == 0) {
            const int64_t o = (int64_t)bh * N + n;
            a.nu[o] = nu + __log2f(tau);  // with tau = 1: the weights are normalised by nu alone
            a.tau[o] = 1.0f;
            a.del[o] = pg / tau;
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
template <int D>
__global__ __launch_bounds__(256) void bw_dkdv_bf16(BackwardArgs a) {
    constexpr int KB = D / 16, DB = D / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char bsm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.y, b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = (M + 31) & ~31, MB = Mp / 32;
    const float c = a.c;
    unsigned char* qs = bsm;
    unsigned char* zs = qs + Mp * 2 * D;
    unsigned char* dzs = zs + Mp * 2 * D;
    float* lam = (float*)(dzs + Mp * 2 * D);  // [Mp] mu* + log2 sig* (+inf for padding)
    float* gam = lam + Mp;                     // [Mp]
    stage_rows<D>(qs, (const uint16_t*)a.Q + (int64_t)h * M * D, M, Mp, tid, 256);
    stage_rows<D>(zs, a.Z + (int64_t)bh * M * D, M, Mp, tid, 256);
    stage_rows<D>(dzs, a.dZ + (int64_t)bh * M * D, M, Mp, tid, 256);
    for (int m = tid; m < Mp; m += 256) {
        const int64_t r = (int64_t)bh * M + m;
        lam[m] = m < M ? a.zmu[r] + __log2f(a.zsig[r]) : INFINITY;
        gam[m] = m < M ? a.gam[r] : 0.0f;
    }
    __syncthreads();
    const uint16_t* Kb = (const uint16_t*)a.K + (int64_t)bh * N * D;
    const uint16_t* Vb = (const uint16_t*)a.V + (int64_t)bh * N * D;
    const uint16_t* Gb = (const uint16_t*)a.dY + (int64_t)bh * N * D;
    const int g = lane >> 4, gi = lane & 15;
    const int prow = enc_row_token(l32);
    const int nblk = (N + 31) / 32;
    for (int blk = blockIdx.x * 4 + wave; blk < nblk; blk += gridDim.x * 4) {
        const int n = blk * 32 + l32, nn = min(n, N - 1);
        bf16x8 kop[KB], vop[KB], gop[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t o = (int64_t)nn * D + 16 * kb + 8 * hi;
            kop[kb] = *(const bf16x8*)(Kb + o);
            vop[kb] = *(const bf16x8*)(Vb + o);
            gop[kb] = *(const bf16x8*)(Gb + o);
        }
        const float nu = a.nu[(int64_t)bh * N + nn], del = a.del[(int64_t)bh * N + nn];
        f32x16 dk[DB], dv[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            dk[db] = f32x16{};
            dv[db] = f32x16{};
        }
        for (int mb = 0; mb < MB; ++mb) {
            bf16x8 qa[KB], za[KB], dza[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = tile_off<D>(32 * mb + prow, 2 * kb + hi);
                qa[kb] = *(const bf16x8*)(qs + off);
                za[kb] = *(const bf16x8*)(zs + off);
                dza[kb] = *(const bf16x8*)(dzs + off);
            }
            f32x16 S = mfma(qa[0], kop[0], f32x16{});
            f32x16 GY = mfma(za[0], gop[0], f32x16{});
            f32x16 GV = mfma(dza[0], vop[0], f32x16{});
#pragma unroll
            for (int kb = 1; kb < KB; ++kb) {
                S = mfma(qa[kb], kop[kb], S);
                GY = mfma(za[kb], gop[kb], GY);
                GV = mfma(dza[kb], vop[kb], GV);
            }
            bf16x8 pe[2], pl[2];
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
                const int m0 = 32 * mb + 16 * kp + 8 * hi;
                const f32x4 l0 = *(const f32x4*)(lam + m0), l1 = *(const f32x4*)(lam + m0 + 4);
                const f32x4 g0 = *(const f32x4*)(gam + m0), g1 = *(const f32x4*)(gam + m0 + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 8 * kp + j;
                    const float lj = j < 4 ? l0[j] : l1[j - 4];
                    const float gj = j < 4 ? g0[j] : g1[j - 4];
                    const float xe = fmaf(S[i], c, -lj);
                    // p_dec <= 1 for real latents; the clamp keeps padded
                    // latents (zero rows) finite
                    const float xd = fminf(fmaf(S[i], c, -nu), 0.0f);
                    const float p_e = exp2_fast(xe);
                    const float p_d = exp2_fast(xd);
                    const float dl = p_e * (GV[i] - gj) + p_d * (GY[i] - del);
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
                lds_tr_op2(taddr(qs, 0, db, 0), taddr(qs, 0, db, 1), taddr(qs, 1, db, 0), taddr(qs, 1, db, 1), qt0, qt1);
                lds_tr_op2(taddr(dzs, 0, db, 0), taddr(dzs, 0, db, 1), taddr(dzs, 1, db, 0), taddr(dzs, 1, db, 1), zt0,
                           zt1);
                dk[db] = mfma(qt0, pl[0], dk[db]);
                dk[db] = mfma(qt1, pl[1], dk[db]);
                dv[db] = mfma(zt0, pe[0], dv[db]);
                dv[db] = mfma(zt1, pe[1], dv[db]);
            }
        }
        // register r of lane l: d = 32 db + 8 (r/4) + 4 hi + r%4, token l32
        if (n < N) {
            uint16_t* dK = (uint16_t*)a.dK + ((int64_t)bh * N + n) * D;
            uint16_t* dV = (uint16_t*)a.dV + ((int64_t)bh * N + n) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d0 = 32 * db + 8 * g4 + 4 * hi;
                    u32x2 wk, wv;
                    const bf16x2 k01 = {(__bf16)(a.s * dk[db][4 * g4]), (__bf16)(a.s * dk[db][4 * g4 + 1])};
                    const bf16x2 k23 = {(__bf16)(a.s * dk[db][4 * g4 + 2]), (__bf16)(a.s * dk[db][4 * g4 + 3])};
                    const bf16x2 v01 = {(__bf16)dv[db][4 * g4], (__bf16)dv[db][4 * g4 + 1]};
                    const bf16x2 v23 = {(__bf16)dv[db][4 * g4 + 2], (__bf16)dv[db][4 * g4 + 3]};
                    wk[0] = __builtin_bit_cast(uint32_t, k01);
                    wk[1] = __builtin_bit_cast(uint32_t, k23);
                    wv[0] = __builtin_bit_cast(uint32_t, v01);
                    wv[1] = __builtin_bit_cast(uint32_t, v23);
                    *(u32x2*)(dK + d0) = wk;
                    *(u32x2*)(dV + d0) = wv;
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
template <int D, bool DQ, int MBW>  // MBW: latent blocks per wave at most
__global__ __launch_bounds__(256) void bw_lat_bf16(BackwardArgs a) {
    constexpr int KB = D / 16, DB = D / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char bsm[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hi = lane >> 5, l32 = lane & 31;
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
    const int nmb = MB > wave ? (MB - wave + 3) / 4 : 0;  // this wave's latent blocks
    // per latent (lane column) of each owned block: lambda = mu* + log2 sig*
    // (+inf for padding) and gam
    float lam[MBW], gm[MBW];
    f32x16 acc[MBW][DB];
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
        const int m = 32 * (wave + 4 * j) + l32;
        const int64_t r = (int64_t)bh * M + min(m, M - 1);
        lam[j] = (DQ && m < M) ? a.zmu[r] + __log2f(a.zsig[r]) : INFINITY;
        gm[j] = (DQ && m < M) ? a.gam[r] : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[j][db] = f32x16{};
    }
    const uint16_t* Kb = (const uint16_t*)a.K + (int64_t)bh * N * D;
    const uint16_t* Vb = (const uint16_t*)a.V + (int64_t)bh * N * D;
    const uint16_t* Gb = (const uint16_t*)a.dY + (int64_t)bh * N * D;
    const float* nub = a.nu + (int64_t)bh * N;
    const float* delb = a.del + (int64_t)bh * N;
    const int prow = enc_row_token(l32);
    const int g = lane >> 4, gi = lane & 15;
    for (int t0 = n0; t0 < n1; t0 += 32) {
        const int nv = n1 - t0;  // valid tokens in this sub-block (>= 1)
        const int tn = t0 + min(prow, nv - 1);
        bf16x8 kA[KB], gA[KB], vA[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int64_t o = (int64_t)tn * D + 16 * kb + 8 * hi;
            kA[kb] = *(const bf16x8*)(Kb + o);
            gA[kb] = *(const bf16x8*)(Gb + o);
            if constexpr (DQ) vA[kb] = *(const bf16x8*)(Vb + o);
        }
        // the accumulation's source rows (K for dQ, dY for dZ) in natural
        // order into this wave's tile; rows past the chunk are zero, so their
        // (finite) weights add nothing
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            *(bf16x8*)(tt + tile_off<D>(prow, 2 * kb + hi)) = prow < nv ? (DQ ? kA[kb] : gA[kb]) : zero8();
        // per token (register i: token 16 (i/8) + 8 hi + i%8): nu' and del
        float nur[16], der[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tk = 16 * (i >> 3) + 8 * hi + (i & 7);
            const int tc = t0 + min(tk, nv - 1);
            nur[i] = tk < nv ? nub[tc] : INFINITY;  // +inf: no weight for tokens past the chunk
            der[i] = DQ ? delb[tc] : 0.0f;
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
            lds_tr_op2(taddr(0, db, 0), taddr(0, db, 1), taddr(1, db, 0), taddr(1, db, 1), tA[0][db], tA[1][db]);
#pragma unroll
        for (int j = 0; j < MBW; ++j) {
            if (j >= nmb) break;
            const int mb = wave + 4 * j;
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
                GY = mfma(gA[0], zB[0], f32x16{});
                GV = mfma(vA[0], dzB[0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) {
                    GY = mfma(gA[kb], zB[kb], GY);
                    GV = mfma(vA[kb], dzB[kb], GV);
                }
            }
            bf16x8 pw[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // decode weight Bt[n][m] (0 past the chunk); clamp: padded
                // latents (zero rows) stay finite
                const float p_d = exp2_fast(fminf(fmaf(S[i], c, -nur[i]), 0.0f));
                float w = p_d;
                if constexpr (DQ) {
                    const float p_e = exp2_fast(fmaf(S[i], c, -lam[j]));
                    w = p_e * (GV[i] - gm[j]) + p_d * (GY[i] - der[i]);
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
    // acc[j][db] register r: d = 32 db + 8 (r/4) + 4 hi + r%4, latent column l32
    const float scale = DQ ? a.s : 1.0f;
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
        if (j >= nmb) break;
        const int m = 32 * (wave + 4 * j) + l32;
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

template <int D, int MBW, int WM, int WT>
hipError_t launch_enc(const EncodeArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH), block(64 * WM * WT);
    hipLaunchKernelGGL((encode_partial_bf16<D, MBW, WM, WT>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D, int MBW, int NWV>
hipError_t launch_enc_priv(const EncodeArgs& a, hipStream_t s) {
    dim3 grid(a.C, a.BH), block(64 * NWV);
    hipLaunchKernelGGL((encode_partial_priv_bf16<D, MBW, NWV>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_enc_d(const EncodeArgs& a, hipStream_t s) {
    const EncCfg cfg = enc_cfg_bf16(D, a.Mp / 32);
    if (cfg.wm == 0) {  // private-stream form: cfg.mbw latent blocks per wave, cfg.wt waves
#define FLARE_ENCP_CASE(MBW, NWV) \
    if (cfg.mbw == MBW && cfg.wt == NWV) return launch_enc_priv<D, MBW, NWV>(a, s);
        FLARE_ENCP_CASE(1, 4)
        if constexpr (D <= 64) {
            FLARE_ENCP_CASE(2, 4)
        }
        if constexpr (D == 32) {
            FLARE_ENCP_CASE(3, 4)
            FLARE_ENCP_CASE(4, 4)
        }
#undef FLARE_ENCP_CASE
        return hipErrorInvalidValue;
    }
#define FLARE_ENC_CASE(MBW, WM, WT) \
    if (cfg.mbw == MBW && cfg.wm == WM && cfg.wt == WT) return launch_enc<D, MBW, WM, WT>(a, s);
    FLARE_ENC_CASE(1, 1, 2)
    FLARE_ENC_CASE(1, 2, 2)
    FLARE_ENC_CASE(1, 4, 1)
    FLARE_ENC_CASE(1, 4, 2)
    if constexpr (D == 128) {
        FLARE_ENC_CASE(1, 8, 1)
    } else {
        FLARE_ENC_CASE(1, 8, 2)
        FLARE_ENC_CASE(2, 4, 1)
        FLARE_ENC_CASE(2, 2, 1)
        FLARE_ENC_CASE(2, 2, 2)
        FLARE_ENC_CASE(2, 1, 2)
        FLARE_ENC_CASE(2, 8, 1)
    }
#undef FLARE_ENC_CASE
    return hipErrorInvalidValue;
}

template <int D, int TB, typename ZT>
const void* dec_kernel(int Mp) {
    if constexpr (D <= 64 && TB == 1) {
        if (Mp > 256) return (const void*)decode_bf16<D, TB, ZT, true>;
    }
    return (const void*)decode_bf16<D, TB, ZT, false>;
}

template <int D, int TB, typename ZT>
hipError_t launch_dec_tb(const DecodeArgs& a, hipStream_t s) {
    const int lds = dec_lds_bytes_bf16(a.Mp, D);
    const void* fn = dec_kernel<D, TB, ZT>(a.Mp);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    DecodeArgs arg = a;
    void* args[] = {&arg};
    hipError_t e = hipLaunchKernel(fn, dim3(a.G, a.BH), dim3(64 * kDecWaves), args, lds, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

template <int D, typename ZT>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t s) {
    if constexpr (D <= 64) {
        if (dec_tb_bf16(D, a.Mp) == 2) return launch_dec_tb<D, 2, ZT>(a, s);
    }
    return launch_dec_tb<D, 1, ZT>(a, s);
}

}  // namespace

EncCfg enc_cfg_bf16(int D, int Mb) {
    // Tuning override (tests and sweeps): "mbw,wm,wt"; must name an
    // instantiated shape that covers Mb latent blocks.
    if (const char* e = std::getenv("FLARE_TEST_ENC_CFG")) {
        int x = 0, y = 0, z = 0;
        if (std::sscanf(e, "%d,%d,%d", &x, &y, &z) == 3 && (y == 0 ? x >= Mb : x * y >= Mb)) return {x, y, z};
    }
    // one latent block: private streams; more: shared tiles (measured equal
    // or faster on MI355X for 2-8 blocks)
    if (Mb <= 1) return {1, 0, 4};
    if (Mb <= 2) return {1, 2, 2};
    if (D == 128) return Mb <= 4 ? EncCfg{1, 4, 1} : EncCfg{1, 8, 1};
    if (Mb <= 4) return {2, 2, 2};
    if (Mb <= 8) return {2, 4, 1};
    return {2, 8, 1};
}

int enc_tile_tokens_bf16(EncCfg cfg) { return cfg.wm == 0 ? 32 * cfg.wt : 64; }
int enc_threads_bf16(EncCfg cfg) { return 64 * (cfg.wm == 0 ? 1 : cfg.wm) * cfg.wt; }

int dec_wgs_per_cu_bf16(int D, int Mp, bool z_f32) {
    const int tb = dec_tb_bf16(D, Mp);
    const int lds = dec_lds_bytes_bf16(Mp, D);
    const void* fn = nullptr;
#define FLARE_DEC_FN(DD, TB)                                                                          \
    if (D == DD && tb == TB) fn = z_f32 ? dec_kernel<DD, TB, float>(Mp) : dec_kernel<DD, TB, uint16_t>(Mp);
    FLARE_DEC_FN(32, 1)
    FLARE_DEC_FN(32, 2)
    FLARE_DEC_FN(64, 1)
    FLARE_DEC_FN(64, 2)
    FLARE_DEC_FN(128, 1)
#undef FLARE_DEC_FN
    if (!fn) return 1;
    if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return 1;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * kDecWaves, lds) != hipSuccess || n < 1) return 1;
    return n;
}

int dec_tb_bf16(int D, int Mp) {
    // Tuning override (tests and sweeps): 32-token blocks per wave and step
    // (2 is built for D <= 64 and M <= 256 only).
    if (const char* e = std::getenv("FLARE_TEST_DEC_TB")) {
        const int v = std::atoi(e);
        if (v == 1 || (v == 2 && D <= 64 && Mp <= 256)) return v;
    }
    // one block: fewer registers, more resident waves (measured faster on
    // MI355X than two at D = 32, equal or faster at D = 64)
    return 1;
}

int dec_lds_bytes_bf16(int Mp, int D) { return Mp * 2 * D + D * (2 * Mp + 16) + 64; }

bool bw_bf16_fits(int M, int D) {
    // Q, Z and dZ of the head (and small per-latent or per-wave buffers) in
    // one CU's LDS; at D = 64 up to M = 256
    const int Mp = (M + 31) / 32 * 32;
    return (D == 32 || (D == 64 && Mp <= 256)) && 3 * Mp * 2 * D + 4 * 32 * 2 * D + 8 * Mp <= 163840;
}

namespace {
template <typename F>
hipError_t launch_bw_tok(F fn, const BackwardArgs& a, int lds, hipStream_t s) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    const int nblk = (a.N + 31) / 32;
    int G = (1024 + a.BH - 1) / a.BH;
    G = std::max(1, std::min(G, (nblk + 3) / 4));
    hipLaunchKernelGGL(fn, dim3(G, a.BH), dim3(256), lds, s, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_bw_stats_bf16(const BackwardArgs& a, hipStream_t s) {
    const int Mp = (a.M + 31) / 32 * 32, lds = 2 * Mp * 2 * a.D;
    if (a.D == 32) return launch_bw_tok(bw_stats_bf16<32>, a, lds, s);
    if (a.D == 64) return launch_bw_tok(bw_stats_bf16<64>, a, lds, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bw_lat_bf16(const BackwardArgs& a, bool dq, hipStream_t s) {
    const int Mp = (a.M + 31) / 32 * 32;
    const int lds = (dq ? 3 : 1) * Mp * 2 * a.D + 4 * 32 * 2 * a.D;
    auto go = [&](auto fn) -> hipError_t {
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(fn, dim3(a.C, a.BH), dim3(256), lds, s, a);
        return hipGetLastError();
    };
    const bool wide = Mp > 256;  // more than 2 latent blocks per wave
    if (a.D == 32) {
        if (wide) return dq ? go(bw_lat_bf16<32, true, 4>) : go(bw_lat_bf16<32, false, 4>);
        return dq ? go(bw_lat_bf16<32, true, 2>) : go(bw_lat_bf16<32, false, 2>);
    }
    if (a.D == 64 && !wide) return dq ? go(bw_lat_bf16<64, true, 2>) : go(bw_lat_bf16<64, false, 2>);
    return hipErrorInvalidValue;
}

hipError_t launch_bw_dkdv_bf16(const BackwardArgs& a, hipStream_t s) {
    const int Mp = (a.M + 31) / 32 * 32, lds = 3 * Mp * 2 * a.D + 8 * Mp;
    if (a.D == 32) return launch_bw_tok(bw_dkdv_bf16<32>, a, lds, s);
    if (a.D == 64) return launch_bw_tok(bw_dkdv_bf16<64>, a, lds, s);
    return hipErrorInvalidValue;
}

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
