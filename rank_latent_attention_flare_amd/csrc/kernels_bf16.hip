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
#include <atomic>
#include <mutex>
#include <vector>
#include <type_traits>

#include "launch.h"

namespace flare {
namespace {

#include "gfx950_ops.h"

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

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1, so that the
// index is a constant expression inside f.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// lds_tr_op2 with constant instruction offsets: operand 1 from a1 + O1 and
// a2 + O1, operand 2 from a3 + O2 and a4 + O2 (LDS byte addresses). Waits for
// its own results, as lds_tr_op2 does.
template <int O1, int O2>
__device__ __forceinline__ void lds_tr_op2_imm(uint32_t a1, uint32_t a2, uint32_t a3, uint32_t a4, bf16x8& o1,
                                               bf16x8& o2) {
    static_assert(O1 >= 0 && O1 < 65536 && O2 >= 0 && O2 < 65536, "LDS instruction offset range");
    u32x2 w1, w2, w3, w4;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%9\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w1), "=&v"(w2), "=&v"(w3), "=&v"(w4)
        : "v"(a1), "v"(a2), "v"(a3), "v"(a4), "i"(O1), "i"(O2)
        : "memory");
    const u32x4 x = {w1[0], w1[1], w2[0], w2[1]};
    const u32x4 y = {w3[0], w3[1], w4[0], w4[1]};
    o1 = __builtin_bit_cast(bf16x8, x);
    o2 = __builtin_bit_cast(bf16x8, y);
}

// 16-byte LDS reads from kofs[i] + O (LDS byte addresses), N at a time, in
// inline asm that waits for its own results. Reads the compiler can see
// after a global->LDS transfer make it wait for every transfer in flight
// (it cannot tell which LDS bytes they write), which would drain the ring.
template <int N, int O>
__device__ __forceinline__ void lds_b128(const uint32_t* addr, bf16x8* r) {
    static_assert(O >= 0 && O < 65536, "LDS instruction offset range");
    if constexpr (N == 2) {
        u32x4 x, y;
        asm volatile(
            "ds_read_b128 %0, %2 offset:%4\n\t"
            "ds_read_b128 %1, %3 offset:%4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x), "=&v"(y)
            : "v"(addr[0]), "v"(addr[1]), "i"(O)
            : "memory");
        r[0] = __builtin_bit_cast(bf16x8, x);
        r[1] = __builtin_bit_cast(bf16x8, y);
    } else {
        static_assert(N % 4 == 0, "reads come in fours");
#pragma unroll
        for (int q = 0; q < N; q += 4) {
            u32x4 x, y, z, w;
            asm volatile(
                "ds_read_b128 %0, %4 offset:%8\n\t"
                "ds_read_b128 %1, %5 offset:%8\n\t"
                "ds_read_b128 %2, %6 offset:%8\n\t"
                "ds_read_b128 %3, %7 offset:%8\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(x), "=&v"(y), "=&v"(z), "=&v"(w)
                : "v"(addr[q]), "v"(addr[q + 1]), "v"(addr[q + 2]), "v"(addr[q + 3]), "i"(O)
                : "memory");
            r[q] = __builtin_bit_cast(bf16x8, x);
            r[q + 1] = __builtin_bit_cast(bf16x8, y);
            r[q + 2] = __builtin_bit_cast(bf16x8, z);
            r[q + 3] = __builtin_bit_cast(bf16x8, w);
        }
    }
}

template <int D, int MBW, int WM, int WT>
struct EncShape {
    static constexpr int KB = D / 16, DB = D / 32, CH = D / 8, RB = 2 * D;
    static constexpr int NW = WM * WT;
    static constexpr int T = 64;
    static constexpr int SB = T / (32 * WT);
    static constexpr int TBY = T * RB;         // one tensor's tile
    static constexpr int SBYTES = 2 * TBY;     // K and V of one stage
    // ring depth: 4 stages of 8 KB tiles (D = 32; measured best on MI355X),
    // otherwise as many stages as fit in 64 KB, at least 3
    static constexpr int NS = SBYTES <= 8192 ? 4 : ((65536 / SBYTES) < 3 ? 3 : ((65536 / SBYTES) > 8 ? 8 : (65536 / SBYTES)));
    static constexpr int PIECES = T * CH / 64;     // 1 KB transfers per tensor per tile
    static constexpr int IPW = PIECES >= NW ? PIECES / NW : 1;  // per issuing wave
    static constexpr int NWI = PIECES / IPW;       // issuing waves: the first NWI
    static constexpr int MERGE_BYTES = (WT - 1) * WM * MBW * (16 * DB + 2) * 64 * 4;
    // LDS: the K tiles of all NS stages, then the V tiles of all stages (so
    // that a stage's offset within either ring fits the 16-bit LDS instruction
    // offset at D = 128 too)
    static constexpr int SMEM = NS * SBYTES > MERGE_BYTES ? NS * SBYTES : MERGE_BYTES;
    static_assert(SB >= 1 && SB * 32 * WT == T, "tile split");
    static_assert(IPW * NWI == PIECES && NWI <= NW, "tile transfer split");
};

template <int D, int MBW, int WM, int WT>
__global__ __launch_bounds__(64 * WM * WT) void encode_partial_bf16(EncodeArgs a) {
    using Sh = EncShape<D, MBW, WM, WT>;
    constexpr int KB = Sh::KB, DB = Sh::DB, CH = Sh::CH, RB = Sh::RB, NW = Sh::NW, T = Sh::T, SB = Sh::SB;
    constexpr int NS = Sh::NS, IPW = Sh::IPW, NWI = Sh::NWI, TBY = Sh::TBY;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sh::SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    const int wm = wave % WM, wt = wave / WM;
    const int chunk = a.heads_fast ? blockIdx.y : blockIdx.x, bh = a.heads_fast ? blockIdx.x : blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int N = a.N, M = a.M, Mp = a.Mp;
    const int n0 = chunk * a.chunk_len;
    const int n1 = min(N, n0 + a.chunk_len);
    const float c = a.c;
    const int64_t kvoff = (int64_t)b * a.sb + (int64_t)h * a.sh;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + kvoff;
    const uint16_t* __restrict__ Vb = (const uint16_t*)a.V + kvoff;
    const uint16_t* __restrict__ Qb = (const uint16_t*)a.Q + (int64_t)b * a.q_bstride + (int64_t)h * M * D;

    // This wave's latent queries as MFMA B operands (column m, k = d). A
    // workgroup covers 32 * WM * MBW latents; grid z selects which (when M
    // needs more than one workgroup's worth).
    const int mgrp = 32 * WM * MBW * blockIdx.z;
    bf16x8 qop[MBW][KB];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int m = mgrp + 32 * (wm * MBW + mb) + l32;
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
    // lane fetches the global chunk that the swizzle places there. Its byte
    // offset from the tile's first token is the same for every full tile, so
    // those need only a wave-uniform base; the ragged last tile clamps rows
    // past the chunk end to its last token (finite data; their logits are
    // masked). Waves that move nothing have no transfers to wait for.
    constexpr bool KNT = D >= 64 && MBW >= 2;
    const bool fixed_off = a.sn < (int64_t(1) << 24);  // T * sn * 2 bytes fit in 32 bits
    uint32_t poff[IPW];
    auto piece = [&](int i, int& row, int& ch) __attribute__((always_inline)) {
        const int p = (i * NWI + wave) * 64 + lane;
        row = p / CH;
        ch = (p % CH) ^ ((tile_off<D>(row, 0) - row * RB) >> 4);
    };
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        int row, ch;
        piece(i, row, ch);
        poff[i] = fixed_off ? (uint32_t)(row * (int)a.sn + ch * 8) * 2u : 0u;
    }
    auto issue = [&](int tile, int stage) __attribute__((always_inline)) {
        if (wave >= NWI) return;
        const int t0 = n0 + tile * T;
        unsigned char* st = smem + stage * TBY;  // K; V at st + NS * TBY
        if (fixed_off && t0 + T <= n1) {
            const unsigned char* kg = (const unsigned char*)(Kb + (int64_t)t0 * a.sn);
            const unsigned char* vg = (const unsigned char*)(Vb + (int64_t)t0 * a.sn);
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int pc = i * NWI + wave;
                // V is read with the non-temporal policy: K, which the decode
                // reads again, then stays in the last-level caches when it
                // fits (measured 7-17% faster decodes on MI355X at 134 MB of
                // K). K is non-temporal too for the D = 64 shapes with two
                // latent blocks per wave (faster there; their K does not fit
                // anyway).
                // (the offset is re-materialised here so that its zero
                // extension stays next to the loads, which then take the
                // uniform base in scalar registers; V goes first so that the
                // compiler does not merge these loads with the clamped ones)
                uint32_t po = poff[i];
                asm volatile("" : "+v"(po));
                dma16<true>(vg + po, st + NS * TBY + pc * 1024);
                dma16<KNT>(kg + po, st + pc * 1024);
            }
            asm volatile("" ::: "memory");
        } else {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int pc = i * NWI + wave;
                int row, ch;
                piece(i, row, ch);
                const int n = min(t0 + row, n1 - 1);
                const int64_t g = (int64_t)n * a.sn + ch * 8;
                dma16<KNT>(Kb + g, st + pc * 1024);
                dma16<true>(Vb + g, st + NS * TBY + pc * 1024);
            }
        }
    };

    const int ntiles = (n1 - n0 + T - 1) / T;
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        if (j < ntiles) issue(j, j);
    // Everything in flight so far (the latent queries and the first tiles,
    // issued back to back) lands together. Waiting for it here, once, leaves
    // the loop with nothing but its own transfers outstanding; otherwise the
    // compiler guards the loop's first use of the queries with a full wait
    // on every pass.
    wait_vmcnt<0>();

    // LDS byte offsets of this lane's operands in stage 0, sub-block 0 of its
    // token group. Stage s, sub-block j and (for V) k-half kp add
    // s*TBY + 32*j*RB + 16*kp*RB: the row swizzle repeats every 16 rows,
    // so those are constants (instruction offsets in the unrolled loop).
    // K rows as A operands of S^T = K Q^T; V^T operands (A of acc^T += V^T
    // P^T; k = 16 tokens) read transposed from the row-major V tile: lane i of
    // each 16-lane group receives element i%4 of source lanes 4k + i/4.
    const int r0 = 32 * wt * SB;
    uint32_t kofs[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kofs[kb] = lds_addr(smem) + tile_off<D>(r0 + enc_row_token(l32), 2 * kb + hi);
    uint32_t vofs[DB][2];
    {
        const int g = lane >> 4, gi = lane & 15;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int second = 0; second < 2; ++second) {
                const int row = r0 + 8 * (g >> 1) + (gi >> 2) + 4 * second;
                const int dcol = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
                vofs[db][second] = lds_addr(smem) + NS * TBY + tile_off<D>(row, dcol >> 3) + ((dcol >> 2) & 1) * 8;
            }
    }

    constexpr bool kLogitsFirst = MBW == 1 && SB > 1 && D == 128;
    // Tile `it` in LDS stage S (a constant) plus sro bytes (0 in the unrolled
    // loop; the stage offset otherwise). tail: the chunk's last, ragged tile,
    // whose sub-blocks may be partial or empty.
    auto tile = [&](int it, bool tail, auto stage_c, int sro) __attribute__((always_inline)) {
        constexpr int S = decltype(stage_c)::value;
        const int valid = n1 - (n0 + it * T);
        // Logits S^T of sub-block j: 32 tokens x (32 * MBW) latents (bf16
        // products, fp32 accumulation), padded tokens masked.
        auto logits = [&](auto jc, f32x16 (&Sx)[MBW]) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            constexpr int SOFF = S * TBY + 32 * j * RB;  // stage and sub-block
            const int nv = valid - 32 * (wt * SB + j);     // valid tokens in this sub-block
            bf16x8 ka[KB];
            uint32_t kad[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kad[kb] = kofs[kb] + sro;
            lds_b128<KB, SOFF>(kad, ka);
            // At D = 32 the wave issues its logit MFMAs at raised priority, so
            // the arbiter takes them ahead of other waves' softmax work
            // (measured 6% faster on MI355X; slower at D = 64).
            if constexpr (D == 32) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                Sx[mb] = mfma(ka[0], qop[mb][0], f32x16{});
#pragma unroll
                for (int kb = 1; kb < KB; ++kb) Sx[mb] = mfma(ka[kb], qop[mb][kb], Sx[mb]);
                if constexpr (D == 32) { if (mb == MBW - 1) __builtin_amdgcn_s_setprio(0); }
                if (tail) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tok = 16 * (i >> 3) + 8 * hi + (i & 7);
                        if (tok >= nv) Sx[mb][i] = -INFINITY;
                    }
                }
            }
        };
        // Softmax of sub-block j against the running offsets, then
        // acc^T += V^T P^T.
        auto update = [&](auto jc, f32x16 (&Sx)[MBW]) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            constexpr int SOFF = S * TBY + 32 * j * RB;
            constexpr int NOP = 2 * DB;
            bf16x8 va[NOP];
            auto read_v = [&]() __attribute__((always_inline)) {
                static_for<0, NOP / 2>([&](auto oc) __attribute__((always_inline)) {
                    constexpr int o = 2 * decltype(oc)::value;
                    constexpr int kp0 = o / DB, db0 = o % DB, kp1 = (o + 1) / DB, db1 = (o + 1) % DB;
                    lds_tr_op2_imm<SOFF + 16 * kp0 * RB, SOFF + 16 * kp1 * RB>(
                        vofs[db0][0] + sro, vofs[db0][1] + sro, vofs[db1][0] + sro, vofs[db1][1] + sro, va[o],
                        va[o + 1]);
                });
            };
            // At D >= 64 the reads are issued first, so their latency overlaps
            // the softmax (measured 3-4% faster on MI355X); at D = 32 after
            // the softmax (faster there).
            constexpr bool kVEarly = D >= 64;
            if constexpr (kVEarly) read_v();
            bf16x8 pb[MBW][2];
            float ts[MBW];
            bool bad = false;
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) exp2_pack(Sx[mb], c, mu[mb], pb[mb][0], pb[mb][1]);
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
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, Sx[mb][i]);
                    const float mnew = fmaxf(mu[mb], pair_max(mx) * c);
                    const float alpha = (mu[mb] == -INFINITY) ? 0.0f : exp2_fast(mu[mb] - mnew);
                    ps[mb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[mb][db] *= alpha;
                    mu[mb] = mnew;
                    exp2_pack(Sx[mb], c, mu[mb], pb[mb][0], pb[mb][1]);
                    ts[mb] = colsum(csel, pb[mb][0], pb[mb][1], f32x4{})[0];
                }
            }
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) ps[mb] += ts[mb];
            if constexpr (!kVEarly) read_v();
#pragma unroll
            for (int o = 0; o < NOP; ++o) {
                const int kp = o / DB, db = o % DB;
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb) acc[mb][db] = mfma(va[o], pb[mb][kp], acc[mb][db]);
            }
        };
        auto live = [&](int j) __attribute__((always_inline)) { return !tail || valid - 32 * (wt * SB + j) > 0; };
        if constexpr (kLogitsFirst) {
            // With one latent block per wave, the logits of every sub-block
            // go to the matrix core before the first softmax, which then runs
            // on the VALU while they complete.
            f32x16 Sx[SB][MBW];
            static_for<0, SB>([&](auto jc) __attribute__((always_inline)) {
                if (live(decltype(jc)::value)) logits(jc, Sx[decltype(jc)::value]);
            });
            static_for<0, SB>([&](auto jc) __attribute__((always_inline)) {
                if (live(decltype(jc)::value)) update(jc, Sx[decltype(jc)::value]);
            });
        } else {
            static_for<0, SB>([&](auto jc) __attribute__((always_inline)) {
                if (!live(decltype(jc)::value)) return;
                f32x16 Sx[MBW];
                logits(jc, Sx);
                update(jc, Sx);
            });
        }
    };
    const bool ragged = (n1 - n0) % T != 0;
    const int nfull = ragged ? ntiles - 1 : ntiles;
    // Tile `it` is complete once at most the transfers of the (up to NS-2)
    // later tiles issued so far are outstanding; then the stage that tile
    // it-1 used is free for tile it+NS-1.
    auto sync_issue = [&](int it) __attribute__((always_inline)) {
        if (it + NS - 2 < ntiles)
            wait_vmcnt<(NS - 2) * 2 * IPW>();
        else
            wait_vmcnt<0>();
        raw_barrier();
        if (it + NS - 1 < ntiles) issue(it + NS - 1, (it + NS - 1) % NS);
    };
    int it = 0;
    // Full tiles NS at a time, each stage's offsets constant (they fit the
    // 16-bit instruction offset); then the rest one at a time.
    constexpr bool kImm = (NS - 1) * TBY + (SB - 1) * 32 * RB + 16 * RB < 65536;
    if constexpr (kImm) {
        for (; it + NS <= nfull; it += NS)
            static_for<0, NS>([&](auto sc) __attribute__((always_inline)) {
                sync_issue(it + decltype(sc)::value);
                tile(it + decltype(sc)::value, false, sc, 0);
            });
    }
    for (; it < ntiles; ++it) {
        sync_issue(it);
        tile(it, it == nfull, std::integral_constant<int, 0>{}, (it % NS) * TBY);
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
        const int64_t pbase = ((int64_t)bh * a.C + chunk) * Mp;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb) {
            const int m = mgrp + 32 * (wm * MBW + mb) + l32;
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
    const int chunk = a.heads_fast ? blockIdx.y : blockIdx.x, bh = a.heads_fast ? blockIdx.x : blockIdx.y;
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
    const int64_t pbase = ((int64_t)bh * a.C + chunk) * Mp;
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
// Workgroup = NW waves for one (b, h); Q[h] (or Q'[b,h]) and Z[b,h] are
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
// MBC > 0: built for exactly M = 32 * MBC latents (no padded block), so that
// the latent loop has no run-time bounds and its blocks schedule freely.
// NW: waves per workgroup, all sharing the workgroup's one LDS copy of Q and
// Z^T. Where that copy is large (D = 64 with M >= 256) more waves per
// workgroup give more resident waves per SIMD than more workgroups could.
// Resident waves per SIMD the register budget is built for.
constexpr int dec_waves_per_simd(int D, int TB, bool LONG, int NW) {
    return (D == 32 && TB == 1 && !LONG) ? 4 : (NW == 12 ? 3 : (NW == 8 ? 2 : 1));
}
// HG: heads per workgroup (a divisor of H). Wave w serves head w % HG of the
// workgroup's group, so the HG waves of one token slot process the same token
// block for HG adjacent heads at the same time: in the token-major layout
// their rows are one contiguous run of HG * D * 2 bytes per token.
// SPLIT (1 or 2): one of the two launches of a decode whose latents do not fit
// in LDS. Each covers the latent range [m_off, m_off + M) of the full a.Mtot,
// against the same kind of offset as the other decodes (the encode's merged
// offsets over that range, else the per-token Cauchy-Schwarz bound), or the
// exact per-token maximum over the range where a sum falls below the floor.
// Launch 1 stores every token's (offset, sum, unnormalised Y) in fp32; launch
// 2 merges its own state with it by the log-sum-exp rule (each side scaled by
// 2^(its offset - the larger offset)) and writes Y.
template <int D, int TB, typename ZT, bool LONG, int MBC = 0, int NW = kDecWaves, int HG = 1, int SPLIT = 0>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(dec_waves_per_simd(D, TB, LONG, NW))))
void decode_bf16(DecodeArgs a) {
    constexpr int KB = D / 16, DB = D / 32, CH = D / 8;
    static_assert(NW >= 1 && NW <= 16, "reduction scratch holds 16 waves");
    static_assert(NW % HG == 0, "every head of the group has the same number of waves");
    static_assert(SPLIT == 0 || (TB == 1 && HG == 1 && MBC == 0), "the split decode is built for one token block");
    const int Mt = SPLIT ? a.Mtot : a.M;  // latents per head in Q and Z (their row stride)
    constexpr int WPH = NW / HG;  // waves (token slots) per head
    const int Mp = a.Mp, MB = Mp / 32;
    const int zs = 2 * Mp + 16;  // bytes per Z^T row (padded)
    const int head_bytes = Mp * 2 * D + D * zs;  // one head's Q and Z^T (a multiple of 16)
    extern __shared__ __attribute__((aligned(16))) unsigned char dsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block indices live in scalar registers
    const int hl = wave % HG, slot = wave / HG;  // this wave's head in the group, and its token slot
    const int hi = lane >> 5, l32 = lane & 31;
    const int ngrp = a.H / HG;
    const int b = blockIdx.y / ngrp, h0 = (blockIdx.y - b * ngrp) * HG;
    const int h = h0 + hl, bh = b * a.H + h;
    const int N = a.N, M = a.M;
    const float c = a.c;
    unsigned char* qs = dsm + hl * head_bytes;  // [Mp][D] bf16, swizzled
    unsigned char* zt = qs + Mp * 2 * D;        // [D][zs bytes]
    float* red = (float*)(dsm + HG * head_bytes);  // [NW] reduction scratch
    const int64_t sn = a.sn;
    const uint16_t* __restrict__ Kb = (const uint16_t*)a.K + (int64_t)b * a.sb + (int64_t)h * a.sh;
    uint16_t* __restrict__ Yb = (uint16_t*)a.Y + (int64_t)b * a.sb + (int64_t)h * a.sh;

    // K rows of one block as MFMA B operands. Rows past the end (the ragged
    // last block, or a block past the wave's last) load the last token
    // instead: every column of the logits belongs to one token, so they only
    // feed outputs that are never stored, and the loads stay unconditional
    // (a fixed number in flight, which the explicit waits below rely on).
    // A lane's byte offset from its block's first token row is the same for
    // every block (when T * sn * 2 bytes fit in 32 bits), so whole blocks are
    // addressed from a uniform base in scalar registers.
    const bool fixed_off = sn < (int64_t(1) << 24);
    uint32_t roff[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) roff[tb] = fixed_off ? (uint32_t)((32 * tb + l32) * (int)sn + 8 * hi) * 2u : 0u;
    auto kload = [&](int bk, bf16x8 (&dst)[TB][KB]) {
        const int nb = bk * 32 * TB;
        if (fixed_off && nb + 32 * TB <= N) {
            const unsigned char* kg = (const unsigned char*)(Kb + (int64_t)nb * sn);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                uint32_t o = roff[tb];
                asm volatile("" : "+v"(o));  // keeps the zero extension next to the loads
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) dst[tb][kb] = *(const bf16x8*)(kg + o + 32 * kb);
            }
            asm volatile("" ::: "memory");
        } else {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int n = min(nb + 32 * tb + l32, N - 1);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    dst[tb][kb] = *(const bf16x8*)(Kb + (int64_t)n * sn + 16 * kb + 8 * hi);
            }
        }
    };
    // This wave's first K block is requested before the staging below, so
    // that its latency overlaps the staging instead of following it.
    int blk = blockIdx.x * WPH + slot;
    bf16x8 kA[TB][KB], kB[TB][KB];
    kload(blk, kA);

    // ---- stage Q (bf16, swizzled rows) and Z^T (bf16, permuted latents) of
    // every head of the group (all threads take part)
    for (int p = tid; p < HG * Mp * CH; p += 64 * NW) {
        const int hh = p / (Mp * CH), r = p - hh * (Mp * CH);
        const int m = r / CH, ch = r % CH;
        const uint16_t* Qh = (const uint16_t*)a.Q + (int64_t)b * a.q_bstride + (int64_t)(h0 + hh) * Mt * D +
                             (int64_t)a.m_off * D;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < M) v = *(const u32x4*)(Qh + (int64_t)m * D + ch * 8);
        *(u32x4*)(dsm + hh * head_bytes + tile_off<D>(m, ch)) = v;
    }
    // four consecutive columns of one latent per thread and step (one 16- or
    // 8-byte load), written to four Z^T rows
    for (int e = tid; e < HG * Mp * (D / 4); e += 64 * NW) {
        const int hh = e / (Mp * (D / 4)), r = e - hh * (Mp * (D / 4));
        const int m = r / (D / 4), d = 4 * (r % (D / 4));
        const ZT* Zh = (const ZT*)a.Z + (int64_t)(b * a.H + h0 + hh) * Mt * D + (int64_t)a.m_off * D;
        float z4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (m < M) {
            if constexpr (sizeof(ZT) == 4) {
                const f32x4 v = *(const f32x4*)((const float*)Zh + (int64_t)m * D + d);
#pragma unroll
                for (int i = 0; i < 4; ++i) z4[i] = v[i];
            } else {
                const u32x2 v = *(const u32x2*)((const uint16_t*)Zh + (int64_t)m * D + d);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    z4[2 * i] = __uint_as_float(v[i] << 16);
                    z4[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
                }
            }
        }
        unsigned char* zh = dsm + hh * head_bytes + Mp * 2 * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(__bf16*)(zh + (d + i) * zs + 2 * dec_zpos(m)) = (__bf16)z4[i];
    }
    __syncthreads();
    // Offsets. With the encode's merged offsets mu*[m] (log2 units), every
    // logit of this (b, h) satisfies c*S <= max_m mu*[m] + 32, one offset for
    // all tokens. Without them, per token: c * max_m |Q[m]| * |K[tok]|
    // (Cauchy-Schwarz); here only max_m |Q[m]|^2 is prepared.
    // (each head's waves reduce over that head's latents)
    const bool goff = a.zmu != nullptr;
    float red_in = goff ? -INFINITY : 0.0f;
    const int ht = lane + 64 * slot;  // this thread's index among its head's threads
    if (goff) {
        for (int m = ht; m < M; m += 64 * WPH) red_in = fmaxf(red_in, a.zmu[(int64_t)bh * Mt + a.m_off + m]);
    } else {
        for (int m = ht; m < M; m += 64 * WPH) {
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
    float rmax = red[hl];
#pragma unroll
    for (int w = hl + HG; w < NW; w += HG) rmax = fmaxf(rmax, red[w]);
    const float cq = goff ? 0.0f : c * sqrtf(rmax);
    const float gnu = goff ? rmax + kSumLimitLog2 : 0.0f;

    const bf16x8 csel = colsum_selector(lane);
    const f32x16 zero16 = {};
    const int nblk = (N + 32 * TB - 1) / (32 * TB);
    const int stride = gridDim.x * WPH;

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
    // normalised, rounded Y of block ypend (-1: none), not yet stored
    bf16x8 ypk[TB][2 * DB];
    int ypend = -1;
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
            const int MBF = MBC > 0 ? MBC : (M >> 5);
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
            if (MBC == 0 && (M & 31)) {
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
        // Exact per-token maxima over the latents, then the sums against them.
        float ex[TB];
        auto exact_run = [&]() {
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
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) ex[tb] = pair_max(mx[tb]) * c;
            run(ex);
        };
        if constexpr (SPLIT > 0) {
            // against the bound first (as below), with exact maxima only when
            // a sum falls below the floor; the state records the offset used
            run(nu);
            float off0 = nu[0];
            if (wave_any(!(tau[0] >= kTauFloor))) {
                exact_run();
                off0 = ex[0];
            }
            // state of token l32 of block bk, in the accumulator's register layout
            const int64_t pb = (int64_t)bh * nblk + bk;
            float* py = a.part_y + pb * (32 * D) + 4 * lane;
            float* pnt = a.part_nt + (pb * 32 + l32) * 2;
            if constexpr (SPLIT == 1) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 v = {yac[0][db][4 * g4], yac[0][db][4 * g4 + 1], yac[0][db][4 * g4 + 2],
                                         yac[0][db][4 * g4 + 3]};
                        *(f32x4*)(py + (db * 4 + g4) * 256) = v;
                    }
                if (hi == 0) {
                    const f32x2 v = {off0, tau[0]};
                    *(f32x2*)pnt = v;
                }
                return;
            } else {
                const f32x2 st = *(const f32x2*)pnt;
                const float nm = fmaxf(st[0], off0);
                const float wa = exp2_fast(st[0] - nm), wb = exp2_fast(off0 - nm);
                const float inv = __builtin_amdgcn_rcpf(fmaf(wa, st[1], wb * tau[0]));
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const f32x4 v = *(const f32x4*)(py + (db * 4 + g4) * 256);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 4 * g4 + i;
                            const float y = fmaf(wa, v[i], wb * yac[0][db][r]) * inv;
                            if (r < 8)
                                ypk[0][2 * db][r] = (__bf16)y;
                            else
                                ypk[0][2 * db + 1][r - 8] = (__bf16)y;
                        }
                    }
                ypend = bk;
                return;
            }
        } else {
            run(nu);
            bool low = false;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) low |= !(tau[tb] >= kTauFloor);
            if (wave_any(low)) exact_run();
        }
        // normalise and round; stored during the next block
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const float inv = __builtin_amdgcn_rcpf(tau[tb]);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    ypk[tb][2 * db][r] = (__bf16)(yac[tb][db][r] * inv);
                    ypk[tb][2 * db + 1][r] = (__bf16)(yac[tb][db][8 + r] * inv);
                }
        }
        ypend = bk;
    };
    // Y rows of block ypend (if any) to memory, 32 bytes per lane and run.
    auto flush = [&]() {
        if (ypend < 0) return;
        const int nb = ypend * 32 * TB;
        if (fixed_off && nb + 32 * TB <= N) {
            unsigned char* yg = (unsigned char*)(Yb + (int64_t)nb * sn);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                uint32_t o = roff[tb] + 16 * hi;  // the row's d = 16*hi.. run (roff holds 8*hi)
                asm volatile("" : "+v"(o));
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    *(bf16x8*)(yg + o + 64 * db) = ypk[tb][2 * db];
                    *(bf16x8*)(yg + o + 64 * db + 16) = ypk[tb][2 * db + 1];
                }
            }
            asm volatile("" ::: "memory");
        } else {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int n = nb + 32 * tb + l32;
                if (n < N) {
                    uint16_t* dst = Yb + (int64_t)n * sn + 16 * hi;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        *(bf16x8*)(dst + 32 * db) = ypk[tb][2 * db];
                        *(bf16x8*)(dst + 32 * db + 8) = ypk[tb][2 * db + 1];
                    }
                }
            }
        }
    };

    // Blocks blk, blk + stride, ... of this wave, with two K register sets in
    // turn. Each step first waits for every memory operation in flight: the
    // K rows of this block and the Y stores of the block before last, both
    // issued one whole block of work earlier. Only then are the next block's
    // K rows requested and the previous block's Y stored, so nothing the step
    // needs is ever behind a transfer issued in the same step. (A wait on a
    // register set alone would also wait for the later loads and the stores:
    // the counter is shared and the compiler takes the conservative count.)
    while (blk < nblk) {
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        kload(blk + stride, kB);
        flush();
        process(blk, kA);
        blk += stride;
        if (blk >= nblk) break;
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        kload(blk + stride, kA);
        flush();
        process(blk, kB);
        blk += stride;
    }
    flush();
}

template <int D, int MBW, int WM, int WT>
hipError_t launch_enc(const EncodeArgs& a, hipStream_t s) {
    const int z = (a.Mp / 32 + MBW * WM - 1) / (MBW * WM);  // latent groups
    dim3 grid(a.heads_fast ? a.BH : a.C, a.heads_fast ? a.C : a.BH, z), block(64 * WM * WT);
    FLARE_LAUNCH((encode_partial_bf16<D, MBW, WM, WT>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D, int MBW, int NWV>
hipError_t launch_enc_priv(const EncodeArgs& a, hipStream_t s) {
    dim3 grid(a.heads_fast ? a.BH : a.C, a.heads_fast ? a.C : a.BH), block(64 * NWV);
    FLARE_LAUNCH((encode_partial_priv_bf16<D, MBW, NWV>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_enc_d(const EncodeArgs& a, hipStream_t s) {
    const EncCfg cfg = a.cfg;
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
const void* dec_kernel(int M, int hg) {
    const int Mp = (M + 31) / 32 * 32;
    if constexpr (D <= 64 && TB == 1) {
        if (hg > 1 && M == Mp) {  // head groups (token-major layout), as dec_heads_bf16 picks them
            if constexpr (D == 32) {
                if (hg == 4) {
                    switch (M / 32) {
                        case 1: return (const void*)decode_bf16<D, TB, ZT, false, 1, 8, 4>;
                        case 2: return (const void*)decode_bf16<D, TB, ZT, false, 2, 8, 4>;
                        case 4: return (const void*)decode_bf16<D, TB, ZT, false, 4, 8, 4>;
                        default: break;
                    }
                } else if (hg == 2 && M == 256) {
                    return (const void*)decode_bf16<D, TB, ZT, false, 8, 8, 2>;
                }
            } else {
                if (hg == 2) {
                    switch (M / 32) {
                        case 1: return (const void*)decode_bf16<D, TB, ZT, false, 1, 4, 2>;
                        case 2: return (const void*)decode_bf16<D, TB, ZT, false, 2, 4, 2>;
                        case 4: return (const void*)decode_bf16<D, TB, ZT, false, 4, 4, 2>;
                        case 8: return (const void*)decode_bf16<D, TB, ZT, false, 8, 12, 2>;
                        default: break;
                    }
                } else if (hg == 4) {
                    switch (M / 32) {
                        case 2: return (const void*)decode_bf16<D, TB, ZT, false, 2, 8, 4>;
                        case 4: return (const void*)decode_bf16<D, TB, ZT, false, 4, 8, 4>;
                        default: break;
                    }
                }
            }
            return nullptr;  // not built
        }
        if (Mp > 256) {
            if constexpr (D == 64)
                return (const void*)decode_bf16<D, TB, ZT, true, 0, 8>;
            else
                return (const void*)decode_bf16<D, TB, ZT, true>;
        }
        if constexpr (D == 64) {
            if (M == 256) return (const void*)decode_bf16<D, TB, ZT, false, 8, 12>;
        }
        if (M == Mp) {
            switch (M / 32) {
                case 1: return (const void*)decode_bf16<D, TB, ZT, false, 1>;
                case 2: return (const void*)decode_bf16<D, TB, ZT, false, 2>;
                case 4: return (const void*)decode_bf16<D, TB, ZT, false, 4>;
                case 8: return (const void*)decode_bf16<D, TB, ZT, false, 8>;
                default: break;
            }
        }
    }
    return (const void*)decode_bf16<D, TB, ZT, false>;
}

// Dynamic LDS above 64 KB must be allowed per kernel (and device) before a
// launch or an occupancy query; done once, for the largest size any plan
// gives a decode kernel.
constexpr int kDecMaxLds = 160 * 1024;
hipError_t allow_dec_lds(const void* fn) {
    struct Done {
        const void* fn;
        int dev;
    };
    static std::mutex mu;
    static std::vector<Done> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    for (const Done& d : done)
        if (d.fn == fn && d.dev == dev) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kDecMaxLds);
    if (e == hipSuccess) done.push_back({fn, dev});
    return e;
}

// The two launches of the split decode (D = 128, M > 256), in workgroups of
// eight waves that share one LDS copy of Q and Z^T (two waves per SIMD where a
// workgroup of four would leave one).
constexpr int kDecSplitWaves = 8;
template <typename ZT>
const void* dec_split_kernel(int split) {
    if (split == 1) return (const void*)decode_bf16<128, 1, ZT, false, 0, kDecSplitWaves, 1, 1>;
    return (const void*)decode_bf16<128, 1, ZT, false, 0, kDecSplitWaves, 1, 2>;
}

template <int D, int TB, typename ZT>
const void* dec_fn(int M, int hg, int split) {
    if constexpr (D == 128 && TB == 1) {
        if (split) return dec_split_kernel<ZT>(split);
    }
    if (split) return nullptr;
    return dec_kernel<D, TB, ZT>(M, hg);
}

template <int D, int TB, typename ZT>
hipError_t launch_dec_tb(const DecodeArgs& a, hipStream_t s) {
    const int lds = dec_lds_bytes_bf16(a.Mp, D, a.hg);
    const void* fn = dec_fn<D, TB, ZT>(a.M, a.hg, a.split);
    if (!fn) return hipErrorInvalidValue;
    if (lds > 65536) {
        hipError_t e = allow_dec_lds(fn);
        if (e != hipSuccess) return e;
    }
    DecodeArgs arg = a;
    void* args[] = {&arg};
    return launch_raw(fn, dim3(a.G, a.BH / a.hg), dim3(64 * dec_waves_bf16(D, a.M, TB, a.hg, a.split)), args, lds, s);
}

template <int D, typename ZT>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t s) {
    if constexpr (D <= 64) {
        if (a.tb == 2) return launch_dec_tb<D, 2, ZT>(a, s);
    }
    return launch_dec_tb<D, 1, ZT>(a, s);
}

}  // namespace

EncCfg enc_cfg_bf16(int D, int Mb) {
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

// Resident decode workgroups per CU, from the kernel's occupancy at its LDS
// size. Computed once per (D, tb, Z type, Mp) and cached: the query and the
// attribute call cost more than a launch.
int dec_wgs_per_cu_bf16(int D, int M, int tb, bool z_f32, int hg, int split) {
    const int di = D == 32 ? 0 : D == 64 ? 1 : D == 128 ? 2 : -1;
    const int hi = hg == 1 ? 0 : hg == 2 ? 1 : hg == 4 ? 2 : -1;
    const int Mp = (M + 31) / 32 * 32;
    if (di < 0 || hi < 0 || tb < 1 || tb > 2 || M < 1 || Mp > kBf16MaxM || split < 0 || split > 2) return 1;
    static std::atomic<int> cache[3][2][2][kBf16MaxM / 32][2][3][3];
    std::atomic<int>& slot = cache[di][tb - 1][z_f32 ? 1 : 0][Mp / 32 - 1][M == Mp ? 1 : 0][hi][split];
    const int known = slot.load(std::memory_order_relaxed);
    if (known > 0) return known;
    const int lds = dec_lds_bytes_bf16(Mp, D, hg);
    const void* fn = nullptr;
#define FLARE_DEC_FN(DD, TB)                                                                          \
    if (D == DD && tb == TB)                                                                          \
        fn = z_f32 ? dec_fn<DD, TB, float>(M, hg, split) : dec_fn<DD, TB, uint16_t>(M, hg, split);
    FLARE_DEC_FN(32, 1)
    FLARE_DEC_FN(32, 2)
    FLARE_DEC_FN(64, 1)
    FLARE_DEC_FN(64, 2)
    FLARE_DEC_FN(128, 1)
#undef FLARE_DEC_FN
    if (!fn) return 1;
    if (lds > 65536 && allow_dec_lds(fn) != hipSuccess) return 1;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * dec_waves_bf16(D, M, tb, hg, split), lds) != hipSuccess ||
        n < 1)
        return 1;
    slot.store(n, std::memory_order_relaxed);
    return n;
}

// One block: fewer registers, more resident waves (measured faster on MI355X
// than two at D = 32, equal or faster at D = 64).
int dec_tb_bf16(int, int) { return 1; }
bool dec_tb_built_bf16(int D, int Mp, int tb) { return tb == 1 || (tb == 2 && D <= 64 && Mp <= 256); }

int dec_waves_bf16(int D, int M, int tb, int hg, int split) {
    const int Mp = (M + 31) / 32 * 32;
    if (split) return kDecSplitWaves;
    if (hg == 4) return 8;                  // two token slots of four heads
    if (hg == 2) return D == 32 ? 8 : (M == 256 ? 12 : kDecWaves);
    if (D != 64 || tb != 1) return kDecWaves;
    if (Mp > 256) return 8;
    return M == 256 ? 12 : kDecWaves;
}

// Head groups built (D, exact M -> hg): D = 32: 4 at M <= 128, 2 at 256;
// D = 64: 2 at M <= 256, 4 at M = 64 and 128.
bool dec_heads_built_bf16(int D, int M, int hg) {
    const int Mp = (M + 31) / 32 * 32;
    if (M != Mp) return hg == 1;
    if (hg == 1) return true;
    if (D == 32) return (hg == 4 && Mp <= 128) || (hg == 2 && Mp == 256);
    if (D == 64) return (hg == 2 && Mp <= 256) || (hg == 4 && (Mp == 64 || Mp == 128));
    return false;
}

// Measured on MI355X in the token-major layout (decode us, heads per
// workgroup 1 / 2 / 4): D = 64, M = 128: 324 / 302 / 275 (FLARE++ workload);
// D = 64, M = 64: 48.1 / 49.6 / 54.4 (long sequences); D = 32, M = 128:
// 55.4 / 56.6 / 56.7 (65k mesh). So: four heads at D = 64, M = 128, pairs at
// D = 64, M = 256 (twelve-wave workgroups), one otherwise.
int dec_heads_bf16(int D, int M, int H, int tb, bool token_major) {
    if (!token_major || tb != 1) return 1;
    int hg = 1;
    if (D == 64 && M == 128) hg = 4;
    else if (D == 64 && M == 256) hg = 2;
    while (hg > 1 && H % hg) hg /= 2;
    return dec_heads_built_bf16(D, M, hg) ? hg : 1;
}

int dec_lds_bytes_bf16(int Mp, int D, int hg) { return hg * (Mp * 2 * D + D * (2 * Mp + 16)) + 64; }

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
