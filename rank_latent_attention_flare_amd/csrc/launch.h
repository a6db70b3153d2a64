// Internal interface between the host runtime (flare.cpp) and the gfx950
// kernels (kernels_bf16.hip, kernels_common.hip, kernels_backward.hip). Not part
// of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flare {

// Every kernel launch of the library goes through launch_raw (flare.cpp):
// hipLaunchKernel, or, while kernel timing is on (flare_timing_enable),
// hipExtLaunchKernel with a HIP event pair bound to the dispatch itself, so
// that the events carry the kernel's own start and end times.
hipError_t launch_raw(const void* fn, dim3 grid, dim3 block, void** args, size_t shm, hipStream_t s);

template <class T>
struct ident {
    using type = T;
};
// Typed front end: the arguments are converted to the kernel's parameter
// types before their addresses are handed to the runtime.
template <typename... P>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shm, hipStream_t s,
                  typename ident<P>::type... args) {
    void* ptrs[] = {(void*)&args..., nullptr};
    return launch_raw((const void*)kernel, grid, block, ptrs, shm, s);
}
// In a function returning hipError_t: launch, and return the error if any.
#define FLARE_LAUNCH(...)                                  \
    do {                                                   \
        const hipError_t flare_e_ = ::flare::launch(__VA_ARGS__); \
        if (flare_e_ != hipSuccess) return flare_e_;       \
    } while (0)

// Encode configuration for bf16. wm > 0: shared-tile form with wm waves over
// latent blocks (mbw blocks each) x wt waves over tokens. wm == 0: private-
// stream form, wt waves that each own all mbw latent blocks.
struct EncCfg {
    int mbw, wm, wt;
};

// Where the split-N encode writes its per-chunk online-softmax state.
struct Partials {
    float* acc;  // [BH][C][Mp][D] unnormalised sums of p * V
    float* mu;   // [BH][C][Mp]    offsets (log2 units) the sums are taken against
    float* sig;  // [BH][C][Mp]    sums of p
};

struct EncodeArgs {
    const void* Q;       // [H][M][D] or, with q_bstride > 0, [B][H][M][D]
    int64_t q_bstride;   // elements between batch entries of Q (0: shared)
    const void* K;       // [B][H][N][D] or [B][N][H][D] (strides below)
    const void* V;       // same layout as K
    int64_t sb, sh, sn;  // K and V strides in elements: batch, head, token
    int BH, H, N, M, Mp, D;
    int C, chunk_len;    // chunks per (b, h) and tokens per chunk
    float c;             // (1/sqrt(D)) * log2(e)
    Partials out;
    EncCfg cfg;          // bf16: the workgroup shape (from the plan)
    bool heads_fast;     // grid (BH, C) instead of (C, BH): adjacent heads' workgroups are dispatched together
};

// What the combine writes.
enum CombineMode {
    COMBINE_Z_F32 = 0,    // fp32 Z [BH][M][D]
    COMBINE_Z_DTYPE = 1,  // Z in the operator dtype [BH][M][D]
    COMBINE_QPRIME = 2    // Q' = Q + Z in the operator dtype [BH][M][D]
};

struct CombineArgs {
    Partials in;
    int BH, H, M, Mp, D, C;
    int mode;
    bool bf16;           // operator dtype (for modes 1 and 2)
    const void* Q;       // mode 2: learned queries [H][M][D]
    void* out;
    float* zmu;          // optional [BH][M]: merged offsets mu* (log2 units) per latent
    float* zsig;         // optional [BH][M]: merged sums sig* against mu*
};

// Backward of the FLARE forward. Storage of Q, K, V, dY, dQ, dK, dV is the
// operator dtype; everything else is fp32 workspace.
struct BackwardArgs {
    const void* Q;       // [H][M][D]
    const void* K;       // [B][H][N][D] or [B][N][H][D] (strides below)
    const void* V;
    const void* dY;
    void* dQ;            // [H][M][D]
    void* dK;            // same layout as K
    void* dV;
    int64_t sb, sh, sn;  // K, V, dY, dK, dV strides in elements: batch, head, token
    const float* Z;      // [BH][M][D] forward encode output
    const float* zmu;    // [BH][M] its offsets mu* (log2 units)
    const float* zsig;   // [BH][M] and sums sig*
    float* nu;           // [BH][N] decode softmax maximum per token (log2 units)
    float* tau;          // [BH][N] and sum against it
    float* del;          // [BH][N] <dY, Y> per token
    float* dZ;           // [BH][M][D]
    float* gam;          // [BH][M] <dZ, Z> per latent
    float* part;         // [BH][C][M][D] per-chunk partial sums (dZ, then dQ)
    int BH, H, N, M, D;
    int C, chunk_len;    // token chunks of the latent kernels
    float s, c;          // 1/sqrt(D) and s * log2(e)
    bool bf16;
    bool accum;          // dK, dV are added to what the outputs hold
    bool enc_only;       // matrix-core kernels: the encode's backward alone (dY unused)
};

struct DecodeArgs {
    const void* Q;       // as in EncodeArgs
    int64_t q_bstride;
    const void* K;       // [B][H][N][D] or [B][N][H][D] (strides below)
    const void* Z;       // [BH][M][D], fp32 or operator dtype
    bool z_f32;
    const float* zmu;    // optional [BH][M] (split: [BH][Mtot]) merged encode offsets; null: per-token bound
    void* Y;             // same layout as K
    int64_t sb, sh, sn;  // K and Y strides in elements: batch, head, token
    int BH, H, N, M, Mp, D;
    int G;               // workgroups per (b, h) group of hg heads
    int tb;              // bf16: 32-token blocks per wave and step (1 or 2)
    int hg;              // bf16: heads per workgroup (a divisor of H; 1 unless token-major)
    // Split decode (bf16, D = 128, M > 256): this launch's latent range
    // [m_off, m_off + M) of Mtot, and the fp32 state between the two launches
    int split;           // 0: whole range; 1: first launch; 2: second launch
    int m_off, Mtot;
    float* part_y;       // [BH][ceil(N/32)][32 * D] unnormalised Y of the first range
    float* part_nt;      // [BH][ceil(N/32) * 32][2] its per-token (offset, sum)
    float c;
};

EncCfg enc_cfg_bf16(int D, int Mb);  // the library's choice for Mb latent blocks
int enc_tile_tokens_bf16(EncCfg cfg);
int enc_threads_bf16(EncCfg cfg);

constexpr int kDecWaves = 4;  // waves per decode workgroup (fp32; bf16 default)
// Largest M of the bf16 path: its decode unrolls every latent block. At
// D = 128 the decode's LDS (Q and Z^T of the head) caps M at 256.
constexpr int kBf16MaxM = 512;
constexpr int kBf16MaxM128 = 512;
// At D = 128 the decode's LDS holds Q and Z^T for at most 256 latents; above
// that it runs in two launches over the two latent ranges (split decode).
constexpr int kDecSplitM128 = 256;
int dec_tb_bf16(int D, int Mp);  // 32-token blocks per wave per step (the library's choice)
bool dec_tb_built_bf16(int D, int Mp, int tb);  // whether a decode with tb blocks is built for (D, Mp)
int dec_wgs_per_cu_bf16(int D, int M, int tb, bool z_f32, int hg, int split);  // resident decode workgroups per CU (cached)
int dec_lds_bytes_bf16(int Mp, int D, int hg);
int dec_waves_bf16(int D, int M, int tb, int hg, int split = 0);  // waves per bf16 decode workgroup
// Heads per bf16 decode workgroup: groups of 2 or 4 heads in the token-major
// layout (for the exact latent counts they are built for), 1 otherwise.
int dec_heads_bf16(int D, int M, int H, int tb, bool token_major);
bool dec_heads_built_bf16(int D, int M, int hg);

hipError_t launch_encode_bf16(const EncodeArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
int enc_threads_f32(int M, int D);  // threads per fp32 encode workgroup
int f32_lanes_enc(int M, int D);    // fp32 lanes per latent (encode)
int f32_lanes_dec(int64_t tokens, int D);  // fp32 lanes per token (decode; tokens = N * B * H)
hipError_t launch_encode_f32(const EncodeArgs& a, hipStream_t s);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
// Peak probes over the whole chip (kind 0: bf16 MFMA, 1: v_exp_f32); one
// float per lane to `out` (kProbeLanes lanes: four waves per SIMD of 256 CUs).
constexpr int kProbeLanes = 256 * 4 * 4 * 64;
hipError_t launch_probe(int kind, int iters, float* out, hipStream_t s);
// Streaming read of `bytes` (one float per probe lane to `out`).
hipError_t launch_read(const void* src, size_t bytes, float* out, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// elementwise helpers (bf16 or fp32 storage; sums in fp32, rounded once)
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s);  // bytes % 16 == 0
// One row copy: rows of row_bytes from src (rows src_pitch bytes apart) to
// dst (dst_pitch apart); every size and address a multiple of 4 bytes.
struct CopyRows {
    void* dst;
    const void* src;
    int64_t rows, row_bytes, src_pitch, dst_pitch;
};
constexpr int kMaxCopies = 8;
// n (<= kMaxCopies) independent row copies in one launch (none may overlap
// another's destination)
hipError_t launch_copy_rows(const CopyRows* c, int n, hipStream_t s);
hipError_t launch_widen(const void* src, float* dst, int64_t n, bool bf16, hipStream_t s);
hipError_t launch_batch_sum(void* dst, const void* base, const void* add, int B, int64_t n, bool bf16, hipStream_t s);

bool backward_supports(int D);
hipError_t launch_bw_stats(const BackwardArgs& a, hipStream_t s);
hipError_t launch_bw_dz(const BackwardArgs& a, hipStream_t s);
hipError_t launch_bw_dz_combine(const BackwardArgs& a, hipStream_t s);
hipError_t launch_bw_dkdv(const BackwardArgs& a, hipStream_t s);
hipError_t launch_bw_dq(const BackwardArgs& a, hipStream_t s);
hipError_t launch_bw_dq_combine(const BackwardArgs& a, hipStream_t s);
// matrix-core versions of bw_stats and bw_dkdv (bf16, D in {32, 64}, Q, Z and
// dZ of a head in at most 96 KB of LDS)
bool bw_bf16_fits(int M, int D);
hipError_t launch_bw_stats_bf16(const BackwardArgs& a, hipStream_t s);
hipError_t launch_bw_dkdv_bf16(const BackwardArgs& a, hipStream_t s);
// Workgroups per (b, h) of the token-side kernels when they also form the
// latent-side partials, else 0: the statistics kernel the dZ partials (bf16,
// the full formula, D = 32 with M <= 128 or D = 64 with M <= 64) and the dK/dV
// kernel the dQ partials (bf16, the full formula, D = 32, M <= 128), each into
// that many chunk slots of a.part; the separate latent-side launch is then
// skipped.
int bw_fused_dz_groups(const BackwardArgs& a);
int bw_fused_dq_groups(const BackwardArgs& a);
hipError_t launch_bw_lat_bf16(const BackwardArgs& a, bool dq, hipStream_t s);  // dZ (dq false) or dQ partials
// per token (n of them): merge a second latent range's statistics (nu2, del2)
// into the first's (nu, del), by the log-sum-exp rule
hipError_t launch_bw_stats_merge(float* nu, float* del, const float* nu2, const float* del2, int64_t n,
                                 hipStream_t s);

}  // namespace flare
