// libflare host runtime: argument validation, launch planning, workspace
// layout, kernel dispatch and the C ABI declared in include/flare.h.
//
// Launch sequences (all on the caller's stream):
//   encode      K1 encode partials -> K2 combine (Z in dtype)
//   decode      K3 decode (Z given)
//   forward     K1 -> K2 (fp32 Z) -> K3
//   pp_forward  K1(Q) -> K2 (Q' = Q + Z0) -> K1(Q') -> K2 (fp32 Z) -> K3(Q')
//   pp_queries  K1(Q) -> K2 (Q' = Q + Z0, the output)
// FLARE skill page steps 2-4 and FLARE arXiv abstract (encode/decode);
// FLARE++ skill page "Core Mechanism" and FLARE++ arXiv abstract (Q').
#include "flare.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

namespace {

using flare::CombineArgs;
using flare::DecodeArgs;
using flare::EncodeArgs;

thread_local std::string g_last_error;

flare_status fail(flare_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

flare_status hip_fail(hipError_t e, const char* what) {
    return fail(FLARE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Tuning overrides (flare_set_tuning); 0 = the library's own choice.
std::atomic<int64_t> g_tune[FLARE_TUNE_KEYS];
int64_t tune(flare_tune k) { return g_tune[k].load(std::memory_order_relaxed); }

constexpr int kTargetEncWaves = 2048;  // waves over all encode workgroups
constexpr int kTargetDecWgs = 1024;    // decode workgroups
constexpr int64_t kMaxGridY = 65535;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Plan {
    flare_dtype dt;
    int64_t B, H, N, M, D;
    int BH, Mp;
    int C, chunk_len;  // encode split over N
    int G;             // decode workgroups per (b, h) (fp32; bf16: decode_groups)
    int tb;            // bf16 decode: 32-token blocks per wave and step
    bool dsplit;       // bf16 D = 128 with M > 256: the decode runs as two launches over the latents
    size_t dsplit_bytes, off_dsplit;  // their fp32 state (decode op: at 0; forward ops: at off_dsplit)
    flare::EncCfg cfg; // bf16 encode workgroup shape
    size_t esize;
    size_t off_acc, off_mu, off_sig, off_z, off_zmu, off_qp, total[7];
    size_t off_zsig, off_nu, off_tau, off_del, off_dz, off_gam;  // backward
    bool bsplit;       // backward over latent ranges of bw_range (bf16: D = 64, 256 < Mp <= 512; D = 128, 128 < Mp <= 512)
    int bw_range;      // latents per range of the latent-side kernels (256 at D = 64, 128 at D = 128)
    int kv_range;      // latents per range of the dK/dV kernel (its LDS holds more at D = 128: 192)
    int stats_range;   // > 0: the per-token statistics too, over ranges of this many latents (D = 128, Mp > 256)
    size_t off_bs_nu2, off_bs_del2;  // a later statistics range's per-token results
    size_t off_bs_q, off_bs_z, off_bs_dz, off_bs_mu, off_bs_sig, off_bs_gam, off_bs_dq;  // one range's latent arrays
    float c;
    int64_t sb, sh, sn;  // element strides of K, V and Y: batch, head, token
};

// Token strides of K, V and Y for a layout (Q and Z are always [.][H][M][D]).
flare_status set_layout(Plan* p, flare_layout layout) {
    if (layout == FLARE_LAYOUT_BHND) {
        p->sn = p->D;
        p->sh = p->N * p->D;
        p->sb = p->H * p->N * p->D;
    } else if (layout == FLARE_LAYOUT_BNHD) {
        p->sn = p->H * p->D;
        p->sh = p->D;
        p->sb = p->N * p->H * p->D;
    } else {
        return fail(FLARE_ERR_INVALID_ARG, "bad layout");
    }
    return FLARE_OK;
}

bool supported(flare_dtype dt, int64_t D, int64_t M, std::string* why) {
    if (dt == FLARE_BF16) {
        if (!(D == 32 || D == 64 || D == 128)) {
            *why = "bf16 supports D in {32, 64, 128}";
            return false;
        }
        const int mmax = D == 128 ? flare::kBf16MaxM128 : flare::kBf16MaxM;
        if (M > mmax) {
            *why = "bf16 supports M <= " + std::to_string(mmax) + " at D = " + std::to_string(D);
            return false;
        }
        return true;
    }
    if (!(D == 8 || D == 16 || D == 24 || D == 32 || D == 48 || D == 64 || D == 96 || D == 128)) {
        *why = "fp32 supports D in {8, 16, 24, 32, 48, 64, 96, 128}";
        return false;
    }
    if (M > 4096) {
        *why = "fp32 supports M <= 4096";
        return false;
    }
    return true;
}

// Sizes and type only (no pointers). Returns OK and fills the plan.
flare_status make_plan(int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dt, Plan* p) {
    if (dt != FLARE_F32 && dt != FLARE_BF16) return fail(FLARE_ERR_INVALID_ARG, "dtype must be FLARE_F32 or FLARE_BF16");
    if (B < 1 || H < 1 || N < 1 || M < 1 || D < 1)
        return fail(FLARE_ERR_INVALID_ARG, "B, H, N, M and D must all be >= 1");
    std::string why;
    if (!supported(dt, D, M, &why)) return fail(FLARE_ERR_UNSUPPORTED, why);
    if (B * H > kMaxGridY) return fail(FLARE_ERR_UNSUPPORTED, "B*H must be <= 65535");
    if (N > (int64_t(1) << 30)) return fail(FLARE_ERR_UNSUPPORTED, "N must be <= 2^30");
    const int64_t esz = dt == FLARE_BF16 ? 2 : 4;
    // every tensor byte count must fit comfortably in 63 bits
    const double kv = double(B) * double(H) * double(N) * double(D) * double(esz);
    if (kv > 4.0e18) return fail(FLARE_ERR_INVALID_ARG, "tensor sizes overflow");

    p->dt = dt;
    p->B = B; p->H = H; p->N = N; p->M = M; p->D = D;
    p->sn = D; p->sh = N * D; p->sb = H * N * D;  // [B][H][N][D] unless set_layout says otherwise
    p->BH = int(B * H);
    p->esize = size_t(esz);
    p->c = float((1.0 / std::sqrt(double(D))) * 1.4426950408889634);
    int tile, waves_per_wg;
    if (dt == FLARE_BF16) {
        p->Mp = int((M + 31) / 32 * 32);
        p->cfg = flare::enc_cfg_bf16(int(D), p->Mp / 32);
        // an override must cover the latent blocks (and name a built shape,
        // else the launch fails)
        const flare::EncCfg o{int(tune(FLARE_TUNE_ENC_MBW)), int(tune(FLARE_TUNE_ENC_WM)),
                              int(tune(FLARE_TUNE_ENC_WT))};
        if (o.mbw > 0 && o.wt > 0 && o.wm >= 0 && (o.wm == 0 ? o.mbw : o.mbw * o.wm) >= p->Mp / 32) p->cfg = o;
        tile = flare::enc_tile_tokens_bf16(p->cfg);
        // waves over all workgroups of one chunk (latent groups on grid z)
        const int zg = p->cfg.wm == 0 ? 1 : (p->Mp / 32 + p->cfg.mbw * p->cfg.wm - 1) / (p->cfg.mbw * p->cfg.wm);
        waves_per_wg = flare::enc_threads_bf16(p->cfg) / 64 * zg;
        p->tb = flare::dec_tb_bf16(int(D), p->Mp);
        const int64_t otb = tune(FLARE_TUNE_DEC_TB);
        if (otb > 0 && flare::dec_tb_built_bf16(int(D), p->Mp, int(otb))) p->tb = int(otb);
    } else {
        p->tb = 2;
        p->cfg = flare::EncCfg{0, 0, 0};
        p->Mp = int(M);
        tile = 32;  // chunk granularity (the kernel's 64-token tiles may be partial)
        const int nth = flare::enc_threads_f32(int(M), int(D));
        const int per = nth / flare::f32_lanes_enc(int(M), int(D));
        waves_per_wg = int((M + per - 1) / per) * (nth / 64);
    }
    // Split over N: enough workgroups to fill the chip, but chunks long enough
    // that the partials stay a few percent of the K/V bytes (bf16: 32*Mp
    // tokens). fp32, whose lanes each run a whole latent through every token
    // of their chunk in one serial chain, takes chunks down to 32 tokens: its
    // time is that chain, and its partials are no burden at the sizes it
    // serves.
    const int64_t target_wgs = std::max<int64_t>(1, kTargetEncWaves / waves_per_wg);
    int64_t C = std::max<int64_t>(1, (target_wgs + p->BH - 1) / p->BH);
    const int64_t min_chunk = dt == FLARE_BF16 ? 32 * int64_t(std::min(p->Mp, 256)) : 32;
    const int64_t cmax = std::max<int64_t>(1, N / min_chunk);
    C = std::min(C, cmax);
    if (tune(FLARE_TUNE_CHUNKS) > 0) C = std::min<int64_t>(tune(FLARE_TUNE_CHUNKS), N);
    int64_t chunk = (N + C - 1) / C;
    chunk = (chunk + tile - 1) / tile * tile;
    C = (N + chunk - 1) / chunk;
    p->C = int(C);
    p->chunk_len = int(chunk);
    // decode workgroups per (b, h)
    const int64_t per_wg = 32 * p->tb * (dt == FLARE_BF16 ? flare::dec_waves_bf16(int(D), int(M), p->tb, 1) : flare::kDecWaves);
    int64_t G = std::max<int64_t>(1, (kTargetDecWgs + p->BH - 1) / p->BH);
    G = std::min<int64_t>(G, (N + per_wg - 1) / per_wg);
    p->G = int(G);
    // workspace layout
    const size_t parts = size_t(p->BH) * size_t(C) * size_t(p->Mp);
    size_t off = 0;
    p->off_acc = off; off = align256(off + parts * size_t(D) * 4);
    p->off_mu = off;  off = align256(off + parts * 4);
    p->off_sig = off; off = align256(off + parts * 4);
    const size_t enc_total = off;
    p->off_z = off;   off = align256(off + size_t(p->BH) * size_t(M) * size_t(D) * 4);
    p->off_zmu = off; off = align256(off + size_t(p->BH) * size_t(M) * 4);
    const size_t fwd_total = off;
    p->off_qp = off;  off = align256(off + size_t(p->BH) * size_t(M) * size_t(D) * p->esize);
    p->total[FLARE_OP_ENCODE] = enc_total;
    // split decode state: per token block, 32 * D floats of Y and 32 (max, sum) pairs
    p->dsplit = dt == FLARE_BF16 && D == 128 && p->Mp > flare::kDecSplitM128;
    const size_t nblk = size_t((N + 31) / 32);
    p->dsplit_bytes = p->dsplit ? align256(size_t(p->BH) * nblk * 32 * size_t(D) * 4) +
                                      align256(size_t(p->BH) * nblk * 32 * 2 * 4)
                                : 0;
    p->off_dsplit = off;  // after every forward section (FLARE++'s Q' included)
    p->total[FLARE_OP_DECODE] = p->dsplit_bytes;
    p->total[FLARE_OP_FORWARD] = p->dsplit ? off + p->dsplit_bytes : fwd_total;
    p->total[FLARE_OP_PP_FORWARD] = off + p->dsplit_bytes;
    p->total[FLARE_OP_PP_QUERIES] = enc_total;
    // backward: the forward's sections (encode partials, reused for the dZ and
    // dQ partials; Z and mu*), then sig*, the per-token decode statistics, dZ
    // and gam
    const size_t tok = size_t(p->BH) * size_t(N) * 4, lat = size_t(p->BH) * size_t(M) * 4;
    off = fwd_total;
    p->off_zsig = off; off = align256(off + lat);
    p->off_nu = off;   off = align256(off + tok);
    p->off_tau = off;  off = align256(off + tok);
    p->off_del = off;  off = align256(off + tok);
    p->off_dz = off;   off = align256(off + lat * size_t(D));
    p->off_gam = off;  off = align256(off + lat);
    // bf16 with more latents than one compute unit's LDS holds Q, Z and dZ of
    // (D = 64: 256 < Mp <= 512; D = 128: 128 < Mp <= 512): the latent-side and
    // dK/dV kernels run over latent ranges of at most bw_range, each on
    // compact copies of the range's latent arrays. The per-token statistics
    // take every latent at once where Q and Z of the head fit in LDS, else
    // (D = 128 above 256 latents) ranges of 256 merged per token.
    p->bw_range = D == 128 ? 128 : 256;
    // (192 at D = 128 where that takes fewer dK/dV passes than ranges of 128:
    // each pass reads every token's rows again; A/B on MI355X at M = 512,
    // 6.00 -> 5.69 ms; at M = 256 the extra copies made it 1% slower)
    p->kv_range = D == 128 && (p->Mp + 191) / 192 < (p->Mp + 127) / 128 ? 192 : p->bw_range;
    p->bsplit = dt == FLARE_BF16 && ((D == 64 && p->Mp > 256 && p->Mp <= 512) || (D == 128 && p->Mp > 128 && p->Mp <= 512));
    p->stats_range = p->bsplit && D == 128 && p->Mp > 256 ? 256 : 0;
    if (p->bsplit) {
        const size_t r = size_t(std::max(std::max(p->bw_range, p->kv_range), p->stats_range));
        p->off_bs_q = off;   off = align256(off + size_t(p->H) * r * size_t(D) * p->esize);
        p->off_bs_z = off;   off = align256(off + size_t(p->BH) * r * size_t(D) * 4);
        p->off_bs_dz = off;  off = align256(off + size_t(p->BH) * r * size_t(D) * 4);
        p->off_bs_mu = off;  off = align256(off + size_t(p->BH) * r * 4);
        p->off_bs_sig = off; off = align256(off + size_t(p->BH) * r * 4);
        p->off_bs_gam = off; off = align256(off + size_t(p->BH) * r * 4);
        p->off_bs_dq = off;  off = align256(off + size_t(p->H) * r * size_t(D) * p->esize);
        if (p->stats_range > 0) {
            p->off_bs_nu2 = off;  off = align256(off + tok);
            p->off_bs_del2 = off; off = align256(off + tok);
        }
    }
    p->total[FLARE_OP_BACKWARD] = off;
    p->total[FLARE_OP_PP_BACKWARD] = 0;  // sized by pp_layout
    return FLARE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = uintptr_t(a), y = uintptr_t(b);
    return x < y + nb && y < x + na;
}

flare_status check_ptrs(const Plan& p, flare_op op, const void* Q, const void* K, const void* V, void* Y) {
    if (!Q || !K || !Y || (op != FLARE_OP_DECODE && !V) || (op == FLARE_OP_DECODE && !V))
        return fail(FLARE_ERR_INVALID_ARG, "null tensor pointer");
    const void* ptrs[4] = {Q, K, V, Y};
    for (const void* q : ptrs)
        if (uintptr_t(q) % 16 != 0) return fail(FLARE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const size_t e = p.esize;
    const size_t nq = size_t(p.H) * p.M * p.D * e;
    const size_t nkv = size_t(p.BH) * p.N * p.D * e;
    const size_t nz = size_t(p.BH) * p.M * p.D * e;
    const size_t nv = op == FLARE_OP_DECODE ? nz : nkv;
    const size_t ny = (op == FLARE_OP_ENCODE || op == FLARE_OP_PP_QUERIES) ? nz : nkv;
    if (overlaps(Y, ny, Q, nq) || overlaps(Y, ny, K, nkv) || overlaps(Y, ny, V, nv))
        return fail(FLARE_ERR_INVALID_ARG, "output overlaps an input");
    return FLARE_OK;
}

// ------------------------------------------------------------------ timing
// While timing is on, every kernel is launched with hipExtLaunchKernel and a
// pair of events bound to its dispatch (the events then hold the kernel's own
// start and end, as a kernel trace shows them), tagged with the kind the
// calling launcher set in t_kind. With timing off the launch path reads one
// atomic flag and takes no lock.
struct Timing {
    std::mutex mu;
    std::atomic<bool> on{false};
    struct Rec {
        int kind;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
};
Timing g_timing;
thread_local int t_kind = -1;

hipEvent_t take_event() {
    if (!g_timing.pool.empty()) {
        hipEvent_t e = g_timing.pool.back();
        g_timing.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <class F>
hipError_t timed(int kind, hipStream_t, F&& launch) {
    t_kind = kind;
    const hipError_t e = launch();
    t_kind = -1;
    return e;
}

// --------------------------------------------------------------- launchers
hipError_t run_encode_partial(const Plan& p, const void* Q, int64_t q_bstride, const void* K, const void* V,
                              char* ws, hipStream_t s) {
    EncodeArgs a{};
    a.Q = Q;
    a.q_bstride = q_bstride;
    a.K = K;
    a.V = V;
    a.sb = p.sb; a.sh = p.sh; a.sn = p.sn;
    a.BH = p.BH; a.H = int(p.H); a.N = int(p.N); a.M = int(p.M); a.Mp = p.Mp; a.D = int(p.D);
    a.C = p.C;
    a.chunk_len = p.chunk_len;
    a.c = p.c;
    a.cfg = p.cfg;
    // Token-major with rows of whole 128-byte lines (D >= 64 in bf16):
    // adjacent heads' workgroups go out together, so that their reads of the
    // same tokens fall on the same DRAM pages at about the same time (the
    // chunk index then takes grid y). With narrower rows two heads share a
    // line, and the chunk-fastest order keeps all heads of a chunk on one
    // XCD and its L2 (the hardware deals workgroups to the 8 XCDs in turn):
    // measured on MI355X, heads first made the D = 64 FLARE++ encode 12%
    // faster and the D = 32 encode 55% slower.
    a.heads_fast = p.sn != p.D && p.D * int64_t(p.esize) >= 128 && p.C <= kMaxGridY;
    a.out.acc = (float*)(ws + p.off_acc);
    a.out.mu = (float*)(ws + p.off_mu);
    a.out.sig = (float*)(ws + p.off_sig);
    return timed(0, s, [&] {
        return p.dt == FLARE_BF16 ? flare::launch_encode_bf16(a, s) : flare::launch_encode_f32(a, s);
    });
}

hipError_t run_combine(const Plan& p, int mode, const void* Q, void* out, char* ws, hipStream_t s,
                       float* zmu = nullptr, float* zsig = nullptr) {
    CombineArgs a{};
    a.in.acc = (float*)(ws + p.off_acc);
    a.in.mu = (float*)(ws + p.off_mu);
    a.in.sig = (float*)(ws + p.off_sig);
    a.BH = p.BH; a.H = int(p.H); a.M = int(p.M); a.Mp = p.Mp; a.D = int(p.D); a.C = p.C;
    a.mode = mode;
    a.bf16 = p.dt == FLARE_BF16;
    a.Q = Q;
    a.out = out;
    a.zmu = zmu;
    a.zsig = zsig;
    return timed(1, s, [&] { return flare::launch_combine(a, s); });
}

// Heads per decode workgroup (bf16): groups in the token-major layout.
int dec_heads(const Plan& p) {
    if (p.dt != FLARE_BF16) return 1;
    const int64_t o = tune(FLARE_TUNE_DEC_HEADS);
    if (o > 0 && p.sn != p.D && p.tb == 1 && p.H % o == 0 && flare::dec_heads_built_bf16(int(p.D), int(p.M), int(o)))
        return int(o);
    return flare::dec_heads_bf16(int(p.D), int(p.M), int(p.H), p.tb, p.sn != p.D);
}

// Decode workgroups per group of heads: one resident wave of workgroups over
// the whole chip (from the kernel's occupancy), each looping over token blocks.
int decode_groups(const Plan& p, bool z_f32, int m_range = 0, int split = 0) {
    if (tune(FLARE_TUNE_DEC_GROUPS) > 0) return int(std::min<int64_t>(tune(FLARE_TUNE_DEC_GROUPS), 1 << 20));
    const int Mr = m_range > 0 ? m_range : int(p.M);  // latents of this launch
    if (p.dt != FLARE_BF16) return p.G;
    static std::atomic<int> cus_cache{0};
    int cus = cus_cache.load(std::memory_order_relaxed);
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
        cus_cache.store(cus, std::memory_order_relaxed);
    }
    const int hg = split ? 1 : dec_heads(p);
    const int per_cu = flare::dec_wgs_per_cu_bf16(int(p.D), Mr, p.tb, z_f32, hg, split);
    const int64_t per_wg = 32 * p.tb * (flare::dec_waves_bf16(int(p.D), Mr, p.tb, hg, split) / hg);
    const int64_t groups = p.BH / hg;
    int64_t G = (int64_t(cus) * per_cu + groups - 1) / groups;
    G = std::max<int64_t>(1, std::min<int64_t>(G, (p.N + per_wg - 1) / per_wg));
    return int(G);
}

hipError_t run_decode(const Plan& p, const void* Q, int64_t q_bstride, const void* K, const void* Z, bool z_f32,
                      void* Y, hipStream_t s, const float* zmu = nullptr, char* split_ws = nullptr) {
    if (p.dsplit) {
        // two launches over latents [0, 256) and [256, M), each against its
        // exact per-token maxima, the second merging the first's state
        if (!split_ws) return hipErrorInvalidValue;
        DecodeArgs a{};
        a.Q = Q; a.q_bstride = q_bstride; a.K = K; a.Z = Z; a.z_f32 = z_f32; a.zmu = zmu; a.Y = Y;
        a.sb = p.sb; a.sh = p.sh; a.sn = p.sn;
        a.BH = p.BH; a.H = int(p.H); a.N = int(p.N); a.D = int(p.D);
        a.tb = 1; a.hg = 1; a.c = p.c; a.Mtot = int(p.M);
        const size_t nblk = size_t((p.N + 31) / 32);
        a.part_y = (float*)split_ws;
        a.part_nt = (float*)(split_ws + align256(size_t(p.BH) * nblk * 32 * size_t(p.D) * 4));
        hipError_t e = hipSuccess;
        for (int part = 1; part <= 2 && e == hipSuccess; ++part) {
            a.split = part;
            a.m_off = part == 1 ? 0 : flare::kDecSplitM128;
            a.M = part == 1 ? flare::kDecSplitM128 : int(p.M) - flare::kDecSplitM128;
            a.Mp = (a.M + 31) / 32 * 32;
            a.G = decode_groups(p, z_f32, a.M, part);
            e = timed(2, s, [&] { return flare::launch_decode_bf16(a, s); });
        }
        return e;
    }
    DecodeArgs a{};
    a.Q = Q;
    a.q_bstride = q_bstride;
    a.K = K;
    a.Z = Z;
    a.z_f32 = z_f32;
    a.zmu = p.dt == FLARE_BF16 ? zmu : nullptr;
    a.Y = Y;
    a.sb = p.sb; a.sh = p.sh; a.sn = p.sn;
    a.BH = p.BH; a.H = int(p.H); a.N = int(p.N); a.M = int(p.M); a.Mp = p.Mp; a.D = int(p.D);
    a.G = decode_groups(p, z_f32);
    a.tb = p.tb;
    a.hg = dec_heads(p);
    a.c = p.c;
    return timed(2, s, [&] {
        return p.dt == FLARE_BF16 ? flare::launch_decode_bf16(a, s) : flare::launch_decode_f32(a, s);
    });
}

flare_status prepare(flare_op op, const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H,
                     int64_t N, int64_t M, int64_t D, flare_dtype dt, flare_layout layout, void* ws, size_t ws_bytes,
                     Plan* p) {
    g_last_error.clear();
    flare_status st = make_plan(B, H, N, M, D, dt, p);
    if (st != FLARE_OK) return st;
    st = set_layout(p, layout);
    if (st != FLARE_OK) return st;
    st = check_ptrs(*p, op, Q, K, V, Y);
    if (st != FLARE_OK) return st;
    const size_t need = p->total[op];
    if (need > 0) {
        if (!ws) return fail(FLARE_ERR_INVALID_ARG, "workspace pointer is null");
        if (uintptr_t(ws) % 256 != 0) return fail(FLARE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(FLARE_ERR_INVALID_ARG,
                        "workspace too small: need " + std::to_string(need) + " bytes, got " + std::to_string(ws_bytes));
    }
    return FLARE_OK;
}

flare_status exec(flare_op op, const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H,
                  int64_t N, int64_t M, int64_t D, flare_dtype dt, flare_layout layout, hipStream_t s, void* wsv,
                  size_t ws_bytes) {
    Plan p;
    flare_status st = prepare(op, Q, K, V, Y, B, H, N, M, D, dt, layout, wsv, ws_bytes, &p);
    if (st != FLARE_OK) return st;
    char* ws = (char*)wsv;
    hipError_t e = hipSuccess;
    switch (op) {
        case FLARE_OP_ENCODE:
            e = run_encode_partial(p, Q, 0, K, V, ws, s);
            if (e == hipSuccess) e = run_combine(p, flare::COMBINE_Z_DTYPE, Q, Y, ws, s);
            break;
        case FLARE_OP_DECODE:
            e = run_decode(p, Q, 0, K, V, dt == FLARE_F32, Y, s, nullptr, ws);
            break;
        case FLARE_OP_PP_QUERIES:
            // the first two launches of pp_forward, with Q' written to the output
            e = run_encode_partial(p, Q, 0, K, V, ws, s);
            if (e == hipSuccess) e = run_combine(p, flare::COMBINE_QPRIME, Q, Y, ws, s);
            break;
        case FLARE_OP_FORWARD:
            e = run_encode_partial(p, Q, 0, K, V, ws, s);
            if (e == hipSuccess)
                e = run_combine(p, flare::COMBINE_Z_F32, Q, ws + p.off_z, ws, s, (float*)(ws + p.off_zmu));
            if (e == hipSuccess)
                e = run_decode(p, Q, 0, K, ws + p.off_z, true, Y, s, (const float*)(ws + p.off_zmu), ws + p.off_dsplit);
            break;
        case FLARE_OP_PP_FORWARD: {
            void* qp = ws + p.off_qp;
            const int64_t qstride = H * M * D;
            e = run_encode_partial(p, Q, 0, K, V, ws, s);
            if (e == hipSuccess) e = run_combine(p, flare::COMBINE_QPRIME, Q, qp, ws, s);
            if (e == hipSuccess) e = run_encode_partial(p, qp, qstride, K, V, ws, s);
            if (e == hipSuccess)
                e = run_combine(p, flare::COMBINE_Z_F32, Q, ws + p.off_z, ws, s, (float*)(ws + p.off_zmu));
            if (e == hipSuccess)
                e = run_decode(p, qp, qstride, K, ws + p.off_z, true, Y, s, (const float*)(ws + p.off_zmu),
                               ws + p.off_dsplit);
            break;
        }
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return FLARE_OK;
}

flare_status exec_alloc(flare_op op, const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H,
                        int64_t N, int64_t M, int64_t D, flare_dtype dt, flare_layout layout, hipStream_t s) {
    Plan p;
    g_last_error.clear();
    flare_status st = make_plan(B, H, N, M, D, dt, &p);
    if (st != FLARE_OK) return st;
    st = set_layout(&p, layout);
    if (st != FLARE_OK) return st;
    st = check_ptrs(p, op, Q, K, V, Y);
    if (st != FLARE_OK) return st;
    const size_t need = p.total[op];
    void* ws = nullptr;
    if (need > 0) {
        if (tune(FLARE_TUNE_FAIL_ALLOC) == 1) return fail(FLARE_ERR_NO_MEMORY, "allocation failure injected (FLARE_TUNE_FAIL_ALLOC)");
        hipError_t e = hipMallocAsync(&ws, need, s);
        if (e != hipSuccess || !ws) return fail(FLARE_ERR_NO_MEMORY, std::string("hipMallocAsync: ") + hipGetErrorString(e));
    }
    st = exec(op, Q, K, V, Y, B, H, N, M, D, dt, layout, s, ws, need);
    if (ws) {
        hipError_t e = hipFreeAsync(ws, s);
        if (e != hipSuccess && st == FLARE_OK) return hip_fail(e, "hipFreeAsync");
    }
    return st;
}

// FLARE++ backward workspace: one FLARE backward's (sized for the whole batch
// and for one batch entry, whichever is larger), then Q' and dQ' [B][H][M][D],
// a zero dY [B][H][N][D] and the first stage's dQ [H][M][D].
struct PPLayout {
    size_t bw, qp, dqp, dy0, dq1, total;
};
PPLayout pp_layout(const Plan& pf, const Plan& p1) {
    PPLayout L{};
    const size_t qm = size_t(pf.BH) * pf.M * pf.D * pf.esize, tok = size_t(pf.BH) * pf.N * pf.D * pf.esize;
    size_t off = align256(std::max(pf.total[FLARE_OP_BACKWARD], p1.total[FLARE_OP_BACKWARD]));
    L.bw = 0;
    L.qp = off;  off = align256(off + qm);
    L.dqp = off; off = align256(off + qm);
    L.dy0 = off; off = align256(off + tok);
    L.dq1 = off; off = align256(off + size_t(pf.H) * pf.M * pf.D * pf.esize);
    L.total = off;
    return L;
}

}  // namespace

namespace {

// Scratch memory of flare_forward_noalloc: a static device array, one copy per
// GPU (the code object's), held until the process ends. Host code never uses
// its name as an address: the device address comes from hipGetSymbolAddress,
// once per device, and is kept per device.
constexpr size_t kStaticScratchBytes = FLARE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device, with that device current).
flare_status static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(FLARE_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || uintptr_t(ptr) % 256 != 0) return fail(FLARE_ERR_HIP, "static scratch has no aligned device address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FLARE_OK;
}

}  // namespace

namespace flare {
hipError_t launch_raw(const void* fn, dim3 grid, dim3 block, void** args, size_t shm, hipStream_t s) {
    if (!g_timing.on.load(std::memory_order_relaxed)) return hipLaunchKernel(fn, grid, block, args, shm, s);
    std::lock_guard<std::mutex> lk(g_timing.mu);
    hipEvent_t a = take_event(), b = take_event();
    if (!a || !b) return hipErrorOutOfMemory;
    const hipError_t e = hipExtLaunchKernel(fn, grid, block, args, shm, s, a, b, 0);
    if (e != hipSuccess) {
        g_timing.pool.push_back(a);
        g_timing.pool.push_back(b);
        return e;
    }
    g_timing.recs.push_back({t_kind, a, b});
    return hipSuccess;
}
}  // namespace flare

extern "C" {

flare_status flare_encode(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                          int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream) {
    return exec_alloc(FLARE_OP_ENCODE, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream);
}
flare_status flare_decode(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                          int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream) {
    return exec_alloc(FLARE_OP_DECODE, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream);
}
flare_status flare_forward(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                           int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream) {
    return exec_alloc(FLARE_OP_FORWARD, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream);
}
flare_status flare_pp_forward(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                              int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream) {
    return exec_alloc(FLARE_OP_PP_FORWARD, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream);
}

size_t flare_workspace_size(flare_op op, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype) {
    if (op < FLARE_OP_ENCODE || op > FLARE_OP_PP_QUERIES) return 0;
    Plan p;
    if (make_plan(B, H, N, M, D, dtype, &p) != FLARE_OK) return 0;
    if (op == FLARE_OP_PP_BACKWARD) {
        Plan p1;
        if (make_plan(1, H, N, M, D, dtype, &p1) != FLARE_OK) return 0;
        return pp_layout(p, p1).total;
    }
    return p.total[op];
}

flare_status flare_encode_ws(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                             int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream, void* ws, size_t n) {
    return exec(FLARE_OP_ENCODE, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, ws, n);
}
flare_status flare_decode_ws(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                             int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream, void* ws, size_t n) {
    return exec(FLARE_OP_DECODE, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, ws, n);
}
flare_status flare_forward_ws(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,
                              int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream, void* ws, size_t n) {
    return exec(FLARE_OP_FORWARD, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, ws, n);
}
flare_status flare_pp_forward_ws(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H,
                                 int64_t N, int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream, void* ws,
                                 size_t n) {
    return exec(FLARE_OP_PP_FORWARD, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, ws, n);
}
flare_status flare_forward_noalloc(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H,
                                   int64_t N, int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream) {
    // Sizes first (no device call), so that an oversized request launches
    // nothing and reports the limit.
    Plan p;
    g_last_error.clear();
    flare_status st = make_plan(B, H, N, M, D, dtype, &p);
    if (st != FLARE_OK) return st;
    const size_t need = p.total[FLARE_OP_FORWARD];
    if (need > kStaticScratchBytes)
        return fail(FLARE_ERR_UNSUPPORTED, "flare_forward_noalloc: workspace of " + std::to_string(need) +
                                               " bytes exceeds the static scratch of " +
                                               std::to_string(kStaticScratchBytes) + " bytes");
    void* ws = nullptr;
    st = static_scratch(&ws);
    if (st != FLARE_OK) return st;
    // The forward writes every workspace byte it later reads (partials, Z,
    // offsets), so nothing needs clearing between calls.
    return exec(FLARE_OP_FORWARD, Q, K, V, Y, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, ws,
                kStaticScratchBytes);
}
flare_status flare_pp_queries(const void* Q, const void* K, const void* V, void* Qp, int64_t B, int64_t H,
                              int64_t N, int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream) {
    return exec_alloc(FLARE_OP_PP_QUERIES, Q, K, V, Qp, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream);
}
flare_status flare_pp_queries_ws(const void* Q, const void* K, const void* V, void* Qp, int64_t B, int64_t H,
                                 int64_t N, int64_t M, int64_t D, flare_dtype dtype, hipStream_t stream, void* ws,
                                 size_t n) {
    return exec(FLARE_OP_PP_QUERIES, Q, K, V, Qp, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, ws, n);
}

}  // extern "C"

namespace {

// Launches of one FLARE backward over a plan's (b, h) problems, in the
// workspace ws (laid out by the plan). With dz_given (the operator dtype,
// [B][H][M][D]) the gradient of Z is that tensor instead of Btᵀ dY: the
// FLARE++ backward uses it, with dY zero, for its first stage (the encode).
hipError_t backward_core(const Plan& p, const void* Q, const void* K, const void* V, const void* dY, void* dQ,
                         void* dK, void* dV, char* ws, hipStream_t s, const void* dz_given, bool accum_kv = false) {
    // forward encode and combine: Z, mu* and sig*
    hipError_t e = run_encode_partial(p, Q, 0, K, V, ws, s);
    if (e == hipSuccess)
        e = run_combine(p, flare::COMBINE_Z_F32, Q, ws + p.off_z, ws, s, (float*)(ws + p.off_zmu),
                        (float*)(ws + p.off_zsig));
    flare::BackwardArgs a{};
    a.Q = Q; a.K = K; a.V = V; a.dY = dY; a.dQ = dQ; a.dK = dK; a.dV = dV;
    a.sb = p.sb; a.sh = p.sh; a.sn = p.sn;
    a.Z = (const float*)(ws + p.off_z);
    a.zmu = (const float*)(ws + p.off_zmu);
    a.zsig = (const float*)(ws + p.off_zsig);
    a.nu = (float*)(ws + p.off_nu);
    a.tau = (float*)(ws + p.off_tau);
    a.del = (float*)(ws + p.off_del);
    a.dZ = (float*)(ws + p.off_dz);
    a.gam = (float*)(ws + p.off_gam);
    a.part = (float*)(ws + p.off_acc);
    a.BH = p.BH; a.H = int(p.H); a.N = int(p.N); a.M = int(p.M); a.D = int(p.D);
    a.C = p.C; a.chunk_len = p.chunk_len;
    a.s = float(1.0 / std::sqrt(double(p.D)));
    a.c = p.c;
    a.bf16 = p.dt == FLARE_BF16;
    a.accum = accum_kv;
    // bf16 heads whose Q, Z and dZ fit in LDS, whole or in latent ranges: the
    // per-token kernels on the matrix core; otherwise (and for fp32) the fp32
    // VALU kernels
    const bool split = p.bsplit;
    const bool mc = a.bf16 && (split || flare::bw_bf16_fits(int(p.M), int(p.D)));
    // With dZ given (the encode's backward alone), the matrix-core kernels
    // skip the decode term and need no per-token statistics; the fp32
    // kernels compute the full formula with the caller's dY = 0.
    a.enc_only = mc && dz_given;
    // bf16 at D = 32 (M <= 128) and D = 64 (M <= 64): the token-side
    // kernels also form the latent-side partials (dZ in the statistics
    // kernel, dQ in the dK/dV kernel), one per workgroup, in fz and fq chunk
    // slots
    const int fz = mc && !split ? flare::bw_fused_dz_groups(a) : 0;
    const int fq = mc && !split ? flare::bw_fused_dq_groups(a) : 0;
    const int64_t M = p.M, D = p.D, H = p.H, BH = p.BH, es = int64_t(p.esize);
    // row copies are collected and issued together, one launch per batch
    flare::CopyRows cp[flare::kMaxCopies];
    int ncp = 0;
    auto rows = [&](void* dst, const void* src, int64_t n, int64_t bytes, int64_t sp, int64_t dp) {
        if (ncp == flare::kMaxCopies && e == hipSuccess) e = hipErrorInvalidValue;
        if (ncp < flare::kMaxCopies) cp[ncp++] = {dst, src, n, bytes, sp, dp};
    };
    auto flush = [&] {
        if (e == hipSuccess && ncp > 0) e = timed(3, s, [&] { return flare::launch_copy_rows(cp, ncp, s); });
        ncp = 0;
    };
    if (e == hipSuccess && !a.enc_only) {
        if (split && p.stats_range > 0) {
            // statistics over latent ranges (compact copies of Q, Z and mu*),
            // the later ones into spare per-token arrays merged into the first
            for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += p.stats_range) {
                const int64_t mr = std::min<int64_t>(p.stats_range, M - m0);
                flare::BackwardArgs sr = a;
                sr.M = int(mr);
                sr.Q = ws + p.off_bs_q;
                sr.Z = (const float*)(ws + p.off_bs_z);
                sr.zmu = (const float*)(ws + p.off_bs_mu);
                if (m0 > 0) {
                    sr.nu = (float*)(ws + p.off_bs_nu2);
                    sr.del = (float*)(ws + p.off_bs_del2);
                }
                rows((void*)sr.Q, (const char*)Q + m0 * D * es, H, mr * D * es, M * D * es, mr * D * es);
                rows((void*)sr.Z, a.Z + m0 * D, BH, mr * D * 4, M * D * 4, mr * D * 4);
                rows((void*)sr.zmu, a.zmu + m0, BH, mr * 4, M * 4, mr * 4);
                flush();
                if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_stats_bf16(sr, s); });
                if (e == hipSuccess && m0 > 0)
                    e = timed(3, s, [&] {
                        return flare::launch_bw_stats_merge(a.nu, a.del, sr.nu, sr.del, BH * int64_t(p.N), s);
                    });
            }
        } else {
            e = timed(3, s, [&] { return mc ? flare::launch_bw_stats_bf16(a, s) : flare::launch_bw_stats(a, s); });
        }
    }
    if (dz_given) {
        // dZ given: one "chunk" of partials holding it, merged as usual
        // (which also forms gam = <dZ, Z>)
        if (e == hipSuccess)
            e = timed(3, s, [&] { return flare::launch_widen(dz_given, a.part, int64_t(p.BH) * p.M * p.D, a.bf16, s); });
        flare::BackwardArgs one = a;
        one.C = 1;
        if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_dz_combine(one, s); });
    } else if (!split) {
        if (e == hipSuccess && fz == 0)
            e = timed(3, s, [&] { return mc ? flare::launch_bw_lat_bf16(a, false, s) : flare::launch_bw_dz(a, s); });
        flare::BackwardArgs dza = a;
        if (fz > 0) dza.C = fz;
        if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_dz_combine(dza, s); });
    }
    if (!split) {
        if (e == hipSuccess)
            e = timed(3, s, [&] { return mc ? flare::launch_bw_dkdv_bf16(a, s) : flare::launch_bw_dkdv(a, s); });
        if (e == hipSuccess && fq == 0)
            e = timed(3, s, [&] { return mc ? flare::launch_bw_lat_bf16(a, true, s) : flare::launch_bw_dq(a, s); });
        flare::BackwardArgs dqa = a;
        if (fq > 0) dqa.C = fq;
        if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_dq_combine(dqa, s); });
        return e;
    }
    // Latent ranges: the range's rows of Q, Z, mu*, sig* (and of a given dZ
    // and its gam) are copied to compact arrays [.][mr][.] (one launch per
    // range for all of its copies), the latent-side
    // kernels and the dK/dV kernel run on them as for a head of mr latents
    // (dK and dV of later ranges added to what the earlier ones wrote), and
    // the range's dQ is copied back into its rows. Where the dK/dV kernel
    // takes larger ranges than the latent kernels (D = 128), the latent loop
    // writes each range's dZ and gam back into the head's arrays, and the
    // dK/dV kernel runs over its own ranges afterwards.
    const bool kv_sep = p.kv_range != p.bw_range;
    auto range_args = [&](int64_t m0, int64_t mr) {
        flare::BackwardArgs ar = a;
        ar.M = int(mr);
        ar.Q = ws + p.off_bs_q;
        ar.Z = (const float*)(ws + p.off_bs_z);
        ar.dZ = (float*)(ws + p.off_bs_dz);
        ar.zmu = (const float*)(ws + p.off_bs_mu);
        ar.zsig = (const float*)(ws + p.off_bs_sig);
        ar.gam = (float*)(ws + p.off_bs_gam);
        ar.dQ = ws + p.off_bs_dq;
        ar.accum = accum_kv || m0 > 0;
        rows((void*)ar.Q, (const char*)Q + m0 * D * es, H, mr * D * es, M * D * es, mr * D * es);
        rows((void*)ar.Z, a.Z + m0 * D, BH, mr * D * 4, M * D * 4, mr * D * 4);
        rows((void*)ar.zmu, a.zmu + m0, BH, mr * 4, M * 4, mr * 4);
        rows((void*)ar.zsig, a.zsig + m0, BH, mr * 4, M * 4, mr * 4);
        return ar;
    };
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += p.bw_range) {
        const int64_t mr = std::min<int64_t>(p.bw_range, M - m0);
        const flare::BackwardArgs ar = range_args(m0, mr);
        if (dz_given) {
            rows(ar.dZ, a.dZ + m0 * D, BH, mr * D * 4, M * D * 4, mr * D * 4);
            rows(ar.gam, a.gam + m0, BH, mr * 4, M * 4, mr * 4);
        }
        flush();
        if (!dz_given) {
            if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_lat_bf16(ar, false, s); });
            if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_dz_combine(ar, s); });
            if (kv_sep) {
                rows(a.dZ + m0 * D, ar.dZ, BH, mr * D * 4, mr * D * 4, M * D * 4);
                rows(a.gam + m0, ar.gam, BH, mr * 4, mr * 4, M * 4);
            }
        }
        const int fqr = kv_sep ? 0 : flare::bw_fused_dq_groups(ar);
        if (e == hipSuccess && !kv_sep) e = timed(3, s, [&] { return flare::launch_bw_dkdv_bf16(ar, s); });
        if (e == hipSuccess && fqr == 0) e = timed(3, s, [&] { return flare::launch_bw_lat_bf16(ar, true, s); });
        flare::BackwardArgs dqa = ar;
        if (fqr > 0) dqa.C = fqr;
        if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_dq_combine(dqa, s); });
        // (with kv_sep, the dZ and gam write-back goes in the same launch)
        rows((char*)dQ + m0 * D * es, ar.dQ, H, mr * D * es, mr * D * es, M * D * es);
        flush();
    }
    for (int64_t m0 = 0; kv_sep && m0 < M && e == hipSuccess; m0 += p.kv_range) {
        const int64_t mr = std::min<int64_t>(p.kv_range, M - m0);
        const flare::BackwardArgs ar = range_args(m0, mr);
        rows(ar.dZ, a.dZ + m0 * D, BH, mr * D * 4, M * D * 4, mr * D * 4);
        rows(ar.gam, a.gam + m0, BH, mr * 4, M * 4, mr * 4);
        flush();
        if (e == hipSuccess) e = timed(3, s, [&] { return flare::launch_bw_dkdv_bf16(ar, s); });
    }
    return e;
}

// Shared argument checks of the backward entry points: null and alignment,
// outputs overlapping inputs or each other.
flare_status check_backward_ptrs(const Plan& p, const void* Q, const void* K, const void* V, const void* dY,
                                 void* dQ, void* dK, void* dV) {
    const void* ins[4] = {Q, K, V, dY};
    void* outs[3] = {dQ, dK, dV};
    for (const void* t : ins)
        if (!t) return fail(FLARE_ERR_INVALID_ARG, "null tensor pointer");
    for (void* t : outs)
        if (!t) return fail(FLARE_ERR_INVALID_ARG, "null tensor pointer");
    for (const void* t : {Q, K, V, dY, (const void*)dQ, (const void*)dK, (const void*)dV})
        if (uintptr_t(t) % 16 != 0) return fail(FLARE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const size_t nq = size_t(p.H) * p.M * p.D * p.esize, nt = size_t(p.BH) * p.N * p.D * p.esize;
    const size_t nin[4] = {nq, nt, nt, nt}, nout[3] = {nq, nt, nt};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlaps(outs[i], nout[i], ins[j], nin[j])) return fail(FLARE_ERR_INVALID_ARG, "output overlaps an input");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], nout[i], outs[j], nout[j])) return fail(FLARE_ERR_INVALID_ARG, "outputs overlap");
    }
    return FLARE_OK;
}

// Workspace: caller's (checked against need) or stream-ordered allocation.
flare_status get_workspace(size_t need, hipStream_t s, void*& wsv, size_t ws_bytes, bool alloc) {
    if (alloc) {
        if (tune(FLARE_TUNE_FAIL_ALLOC) == 1) return fail(FLARE_ERR_NO_MEMORY, "allocation failure injected (FLARE_TUNE_FAIL_ALLOC)");
        hipError_t e = hipMallocAsync(&wsv, need, s);
        if (e != hipSuccess || !wsv) return fail(FLARE_ERR_NO_MEMORY, std::string("hipMallocAsync: ") + hipGetErrorString(e));
        return FLARE_OK;
    }
    if (!wsv) return fail(FLARE_ERR_INVALID_ARG, "workspace pointer is null");
    if (uintptr_t(wsv) % 256 != 0) return fail(FLARE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(FLARE_ERR_INVALID_ARG,
                    "workspace too small: need " + std::to_string(need) + " bytes, got " + std::to_string(ws_bytes));
    return FLARE_OK;
}

flare_status finish(flare_status res, hipError_t e, bool alloc, void* wsv, hipStream_t s) {
    if (res == FLARE_OK && e != hipSuccess) res = hip_fail(e, "kernel launch");
    if (alloc) {
        hipError_t f = hipFreeAsync(wsv, s);
        if (f != hipSuccess && res == FLARE_OK) return hip_fail(f, "hipFreeAsync");
    }
    return res;
}

flare_status backward(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK, void* dV,
                      int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dt, flare_layout layout,
                      hipStream_t s, void* wsv, size_t ws_bytes, bool alloc) {
    Plan p;
    g_last_error.clear();
    flare_status st = make_plan(B, H, N, M, D, dt, &p);
    if (st != FLARE_OK) return st;
    st = set_layout(&p, layout);
    if (st != FLARE_OK) return st;
    if (!flare::backward_supports(int(D)))
        return fail(FLARE_ERR_UNSUPPORTED, "the backward supports D in {8, 16, 24, 32, 48, 64, 96, 128}");
    st = check_backward_ptrs(p, Q, K, V, dY, dQ, dK, dV);
    if (st != FLARE_OK) return st;
    st = get_workspace(p.total[FLARE_OP_BACKWARD], s, wsv, ws_bytes, alloc);
    if (st != FLARE_OK) return st;
    const hipError_t e = backward_core(p, Q, K, V, dY, dQ, dK, dV, (char*)wsv, s, nullptr);
    return finish(FLARE_OK, e, alloc, wsv, s);
}

flare_status pp_backward(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK, void* dV,
                         int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dt, flare_layout layout,
                         hipStream_t s, void* wsv, size_t ws_bytes, bool alloc) {
    Plan pf, p1;
    g_last_error.clear();
    flare_status st = make_plan(B, H, N, M, D, dt, &pf);
    if (st != FLARE_OK) return st;
    st = make_plan(1, H, N, M, D, dt, &p1);
    if (st != FLARE_OK) return st;
    if ((st = set_layout(&pf, layout)) != FLARE_OK || (st = set_layout(&p1, layout)) != FLARE_OK) return st;
    if (!flare::backward_supports(int(D)))
        return fail(FLARE_ERR_UNSUPPORTED, "the backward supports D in {8, 16, 24, 32, 48, 64, 96, 128}");
    st = check_backward_ptrs(pf, Q, K, V, dY, dQ, dK, dV);
    if (st != FLARE_OK) return st;
    const PPLayout L = pp_layout(pf, p1);
    st = get_workspace(L.total, s, wsv, ws_bytes, alloc);
    if (st != FLARE_OK) return st;
    char* ws = (char*)wsv;
    const bool bf = dt == FLARE_BF16;
    // per batch entry (one entry's token rows are contiguous in both layouts)
    const size_t e = pf.esize, qm = size_t(H) * M * D, tok = size_t(H) * N * D;
    // Q' = Q + encode(Q, K, V) for every batch entry
    hipError_t err = run_encode_partial(pf, Q, 0, K, V, ws, s);
    if (err == hipSuccess) err = run_combine(pf, flare::COMBINE_QPRIME, Q, ws + L.qp, ws, s);
    // second stage: the FLARE backward at Q' (one batch entry at a time, its
    // queries being its own), giving dQ' and the second stage's dK, dV
    for (int64_t b = 0; b < B && err == hipSuccess; ++b)
        err = backward_core(p1, ws + L.qp + b * qm * e, (const char*)K + b * tok * e, (const char*)V + b * tok * e,
                            (const char*)dY + b * tok * e, ws + L.dqp + b * qm * e, (char*)dK + b * tok * e,
                            (char*)dV + b * tok * e, ws + L.bw, s, nullptr);
    // first stage: the encode's backward for dZ = dQ' (the FLARE backward with
    // dY = 0 and dZ given); its dK, dV are added to the second stage's in the
    // kernel (fp32 sum, rounded once), its dQ goes to a buffer
    // (the zero dY is read by the fp32 kernels only)
    if (err == hipSuccess && !(bf && (pf.bsplit || flare::bw_bf16_fits(int(M), int(D)))))
        err = flare::launch_fill_zero(ws + L.dy0, size_t(B) * tok * e, s);
    if (err == hipSuccess)
        err = backward_core(pf, Q, K, V, ws + L.dy0, ws + L.dq1, dK, dV, ws + L.bw, s, ws + L.dqp, true);
    // dQ = the first stage's + the sum over the batch of dQ' (fp32, rounded once)
    if (err == hipSuccess) err = flare::launch_batch_sum(dQ, ws + L.dq1, ws + L.dqp, int(B), int64_t(qm), bf, s);
    return finish(FLARE_OK, err, alloc, wsv, s);
}

}  // namespace

extern "C" {

flare_status flare_backward(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK,
                            void* dV, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype,
                            hipStream_t stream) {
    return backward(Q, K, V, dY, dQ, dK, dV, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, nullptr, 0, true);
}

flare_status flare_backward_ws(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK,
                               void* dV, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype,
                               hipStream_t stream, void* workspace, size_t ws_bytes) {
    return backward(Q, K, V, dY, dQ, dK, dV, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, workspace, ws_bytes,
                    false);
}

flare_status flare_pp_backward(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK,
                               void* dV, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype,
                               hipStream_t stream) {
    return pp_backward(Q, K, V, dY, dQ, dK, dV, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, nullptr, 0, true);
}

flare_status flare_pp_backward_ws(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK,
                                  void* dV, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype,
                                  hipStream_t stream, void* workspace, size_t ws_bytes) {
    return pp_backward(Q, K, V, dY, dQ, dK, dV, B, H, N, M, D, dtype, FLARE_LAYOUT_BHND, stream, workspace, ws_bytes,
                       false);
}

flare_status flare_backward_ex(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK,
                               void* dV, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype,
                               flare_layout layout, hipStream_t stream, void* workspace, size_t ws_bytes) {
    const bool alloc = !workspace && ws_bytes == 0;
    return backward(Q, K, V, dY, dQ, dK, dV, B, H, N, M, D, dtype, layout, stream, workspace, ws_bytes, alloc);
}

flare_status flare_pp_backward_ex(const void* Q, const void* K, const void* V, const void* dY, void* dQ, void* dK,
                                  void* dV, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D, flare_dtype dtype,
                                  flare_layout layout, hipStream_t stream, void* workspace, size_t ws_bytes) {
    const bool alloc = !workspace && ws_bytes == 0;
    return pp_backward(Q, K, V, dY, dQ, dK, dV, B, H, N, M, D, dtype, layout, stream, workspace, ws_bytes, alloc);
}

flare_status flare_attend(const void* q, const void* Z, void* Y, int64_t B, int64_t H, int64_t N, int64_t M,
                          int64_t D, flare_dtype dtype, flare_layout layout, hipStream_t stream) {
    Plan p;
    g_last_error.clear();
    flare_status st = make_plan(B, H, N, M, D, dtype, &p);
    if (st != FLARE_OK) return st;
    st = set_layout(&p, layout);
    if (st != FLARE_OK) return st;
    if (!q || !Z || !Y) return fail(FLARE_ERR_INVALID_ARG, "null tensor pointer");
    for (const void* t : {q, Z, (const void*)Y})
        if (uintptr_t(t) % 16 != 0) return fail(FLARE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const size_t ntok = size_t(p.BH) * p.N * p.D * p.esize, nz = size_t(p.BH) * p.M * p.D * p.esize;
    if (overlaps(Y, ntok, q, ntok) || overlaps(Y, ntok, Z, nz))
        return fail(FLARE_ERR_INVALID_ARG, "output overlaps an input");
    // The decode kernel with Z in both latent roles: Z[b][h] is the latent
    // operand of the logits (batch-strided, as FLARE++'s Q') and the values;
    // the token queries take the place of K. No encode offsets: the
    // per-token Cauchy-Schwarz bound.
    // (the split decode needs scratch memory for its state: stream-ordered,
    // as in the plain entry points)
    void* ws = nullptr;
    if (p.dsplit) {
        if (tune(FLARE_TUNE_FAIL_ALLOC) == 1) return fail(FLARE_ERR_NO_MEMORY, "allocation failure injected (FLARE_TUNE_FAIL_ALLOC)");
        hipError_t ea = hipMallocAsync(&ws, p.dsplit_bytes, stream);
        if (ea != hipSuccess || !ws) return fail(FLARE_ERR_NO_MEMORY, std::string("hipMallocAsync: ") + hipGetErrorString(ea));
    }
    hipError_t e = run_decode(p, Z, H * M * D, q, Z, dtype == FLARE_F32, Y, stream, nullptr, (char*)ws);
    if (ws) {
        hipError_t ef = hipFreeAsync(ws, stream);
        if (e == hipSuccess && ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return FLARE_OK;
}

#define FLARE_EX(NAME, OP)                                                                                     \
    flare_status NAME(const void* Q, const void* K, const void* V, void* Y, int64_t B, int64_t H, int64_t N,     \
                      int64_t M, int64_t D, flare_dtype dtype, flare_layout layout, hipStream_t stream, void* ws, \
                      size_t n) {                                                                                 \
        if (!ws && n == 0) return exec_alloc(OP, Q, K, V, Y, B, H, N, M, D, dtype, layout, stream);              \
        return exec(OP, Q, K, V, Y, B, H, N, M, D, dtype, layout, stream, ws, n);                                \
    }
FLARE_EX(flare_encode_ex, FLARE_OP_ENCODE)
FLARE_EX(flare_decode_ex, FLARE_OP_DECODE)
FLARE_EX(flare_forward_ex, FLARE_OP_FORWARD)
FLARE_EX(flare_pp_forward_ex, FLARE_OP_PP_FORWARD)
#undef FLARE_EX

const char* flare_status_string(flare_status s) {
    switch (s) {
        case FLARE_OK: return "FLARE_OK";
        case FLARE_ERR_INVALID_ARG: return "FLARE_ERR_INVALID_ARG";
        case FLARE_ERR_UNSUPPORTED: return "FLARE_ERR_UNSUPPORTED";
        case FLARE_ERR_NO_MEMORY: return "FLARE_ERR_NO_MEMORY";
        case FLARE_ERR_HIP: return "FLARE_ERR_HIP";
    }
    return "FLARE_ERR_UNKNOWN";
}

const char* flare_last_error(void) { return g_last_error.c_str(); }

flare_status flare_set_tuning(flare_tune key, int64_t value) {
    g_last_error.clear();
    if (key < 0 || key >= FLARE_TUNE_KEYS) return fail(FLARE_ERR_INVALID_ARG, "unknown tuning key");
    if (value < 0) return fail(FLARE_ERR_INVALID_ARG, "tuning values are >= 0 (0 = the library's choice)");
    g_tune[key].store(value, std::memory_order_relaxed);
    return FLARE_OK;
}

flare_status flare_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    for (auto& r : g_timing.recs) {
        g_timing.pool.push_back(r.a);
        g_timing.pool.push_back(r.b);
    }
    g_timing.recs.clear();
    g_timing.on.store(on != 0);
    return FLARE_OK;
}

flare_status flare_timing_read(double* ms, int64_t* count) {
    if (!ms || !count) return fail(FLARE_ERR_INVALID_ARG, "null output array");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    flare_status st = FLARE_OK;
    for (auto& r : g_timing.recs) {
        float t = 0.0f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
        if (e != hipSuccess) {
            st = hip_fail(e, "event timing");
        } else if (r.kind >= 0 && r.kind < FLARE_KERNEL_KINDS) {
            ms[r.kind] += double(t);
            count[r.kind] += 1;
        }
        g_timing.pool.push_back(r.a);
        g_timing.pool.push_back(r.b);
    }
    g_timing.recs.clear();
    return st;
}

flare_status flare_copy_kernel(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    g_last_error.clear();
    if (!src || !dst) return fail(FLARE_ERR_INVALID_ARG, "null pointer");
    if (bytes % 16 || uintptr_t(src) % 16 || uintptr_t(dst) % 16)
        return fail(FLARE_ERR_INVALID_ARG, "copy needs 16-byte aligned pointers and size");
    if (overlaps(src, bytes, dst, bytes)) return fail(FLARE_ERR_INVALID_ARG, "copy ranges overlap");
    hipError_t e = flare::launch_copy(src, dst, bytes, stream);
    if (e != hipSuccess) return hip_fail(e, "copy kernel");
    return FLARE_OK;
}

size_t flare_probe_lanes(void) { return size_t(flare::kProbeLanes); }

flare_status flare_read_kernel(const void* src, size_t bytes, float* out, size_t out_floats, hipStream_t stream) {
    g_last_error.clear();
    if (!src || !out) return fail(FLARE_ERR_INVALID_ARG, "null pointer");
    if (bytes % 16 || uintptr_t(src) % 16) return fail(FLARE_ERR_INVALID_ARG, "read needs a 16-byte aligned pointer and size");
    if (out_floats < size_t(flare::kProbeLanes)) return fail(FLARE_ERR_INVALID_ARG, "out holds fewer than flare_probe_lanes() floats");
    const hipError_t e = flare::launch_read(src, bytes, out, stream);
    if (e != hipSuccess) return hip_fail(e, "read kernel");
    return FLARE_OK;
}

flare_status flare_probe_peak(flare_probe kind, int64_t iters, float* out, size_t out_floats, double* work,
                              hipStream_t stream) {
    g_last_error.clear();
    if (kind != FLARE_PROBE_MFMA_BF16 && kind != FLARE_PROBE_EXP) return fail(FLARE_ERR_INVALID_ARG, "bad probe kind");
    if (iters < 1 || iters > (int64_t(1) << 20)) return fail(FLARE_ERR_INVALID_ARG, "iters must be in [1, 2^20]");
    if (!out || !work) return fail(FLARE_ERR_INVALID_ARG, "null pointer");
    if (out_floats < size_t(flare::kProbeLanes)) return fail(FLARE_ERR_INVALID_ARG, "out holds fewer than flare_probe_lanes() floats");
    const double lanes = double(flare::kProbeLanes);
    *work = kind == FLARE_PROBE_MFMA_BF16 ? lanes / 64.0 * double(iters) * 4.0 * 32768.0 : lanes * double(iters) * 16.0;
    const hipError_t e = flare::launch_probe(int(kind), int(iters), out, stream);
    if (e != hipSuccess) return hip_fail(e, "probe kernel");
    return FLARE_OK;
}

flare_status flare_describe_plan(flare_op op, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 flare_dtype dtype, char* buf, size_t len) {
    g_last_error.clear();
    if (!buf || len == 0) return fail(FLARE_ERR_INVALID_ARG, "null buffer");
    if (op < FLARE_OP_ENCODE || op > FLARE_OP_PP_FORWARD) return fail(FLARE_ERR_INVALID_ARG, "bad op");
    Plan p;
    flare_status st = make_plan(B, H, N, M, D, dtype, &p);
    if (st != FLARE_OK) return st;
    std::string enc;
    if (dtype == FLARE_BF16) {
        const flare::EncCfg cfg = p.cfg;
        enc = "encode grid (" + std::to_string(p.C) + "," + std::to_string(p.BH) + ") waves " +
              std::to_string(cfg.wm) + "x" + std::to_string(cfg.wt) + " latent-blocks/wave " + std::to_string(cfg.mbw) +
              " tile " + std::to_string(flare::enc_tile_tokens_bf16(cfg));
    } else {
        const int nth = flare::enc_threads_f32(int(M), int(D)), lanes = flare::f32_lanes_enc(int(M), int(D));
        enc = "encode grid (" + std::to_string(p.C) + "," + std::to_string(p.BH) + "," +
              std::to_string((M + nth / lanes - 1) / (nth / lanes)) + ") threads " + std::to_string(nth) +
              " lanes/latent " + std::to_string(lanes);
    }
    // the launched decode grid (bf16: sized from the device's occupancy)
    const int dec_tpb = 256 / flare::f32_lanes_dec(N * p.BH, int(D));  // fp32: tokens per workgroup
    const int dec_g = dtype == FLARE_BF16 ? decode_groups(p, op != FLARE_OP_DECODE) : int((N + dec_tpb - 1) / dec_tpb);
    std::string txt = enc + " chunk " + std::to_string(p.chunk_len) + "; decode grid (" + std::to_string(dec_g) + "," +
                      std::to_string(p.BH) + "); workspace " + std::to_string(p.total[op]) + " bytes";
    std::snprintf(buf, len, "%s", txt.c_str());
    return FLARE_OK;
}

}  // extern "C"
