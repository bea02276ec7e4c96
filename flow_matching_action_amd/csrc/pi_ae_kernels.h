// Internal interface between the host runtime and the gfx950 kernels of the
// action-expert denoise loop.  Not part of the public C ABI (include/pi_ae.h).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <string>

namespace pi_ae {

// Fixed expert shape (Realtime-VLA technical blog, "LeRobot implementation":
// Gemma-300M-shaped expert, 8 query heads x 256, one KV head, MLP 4096).
constexpr int kD = 1024;              // width
constexpr int kF = 4096;              // MLP dim
constexpr int kH = 8;                 // query heads
constexpr int kHd = 256;              // head dim
constexpr int kA = 32;                // action dim
constexpr int kNqkv = (kH + 2) * kHd; // fused QKV width, 2560
constexpr int kNgu = 2 * kF;          // fused gate|up width, 8192
constexpr int kRopeHalf = kHd / 2;    // 128 rotated pairs per head

// The VLM whose layers fill the prefix KV cache (Realtime-VLA technical blog,
// "pi0.5 inference flow", Encoder phase, and the section 4 encoder kernel
// list: Gemma-2B-shaped, width 2048, fused QKV 2560, MLP 16384; the same 8
// query heads x 256 and one KV head of 256 as the expert reads).
constexpr int kVD = 2048;             // width
constexpr int kVF = 16384;            // MLP dim
constexpr int kVNgu = 2 * kVF;        // fused gate|up width, 32768

// The SigLIP-shaped vision encoder (Realtime-VLA technical blog, "pi0.5
// inference flow" and "LeRobot implementation": 27 layers, 224x224 -> 256
// tokens, width 1152, projector 1152 -> 2048).  GEMM operands are padded to
// whole 256-wide k-blocks with zeros: width inputs 1152 -> 1280, the MLP
// hidden 4304 -> 4352 columns (fc1 output) / 4608 (fc2 input), the patch
// vectors 3 x 14 x 14 = 588 -> 768.
constexpr int kSD = 1152;             // width
constexpr int kSF = 4304;             // MLP dim
constexpr int kSFn = 4352;            // fc1 output columns (padded N)
constexpr int kSFk = 4608;            // fc2 input columns (padded K) = MLP operand stride
constexpr int kSKp = 1280;            // padded K of the width-input GEMMs
constexpr int kSH = 16, kSHd = 72;    // heads x head dim
constexpr int kSPatch = 14, kSImg = 224, kSC = 3;
constexpr int kSTok = (kSImg / kSPatch) * (kSImg / kSPatch);  // 256 tokens per view
constexpr int kSKpatch = 768;         // padded patch vector (588)
constexpr int kSOut = 2048;           // projector output (the VLM width)

// Per-call pointers, written by the args kernel into a device block that the
// captured graph reads, so that one graph serves every call.
struct DevArgs {
  const uint16_t* pk;     // prefix K [L][B][P][256]
  const uint16_t* pv;     // prefix V [L][B][P][256]
  const uint8_t* mask;    // [B][P] or null
  const float* noise;     // [B][T][32]
  float* actions;         // [B][T][32], the Euler state x
};

// From this many rows on the GEMMs are MFMA-bound and use 128 x 128 tiles
// staged through LDS; below it they stream weights with one row tile.
constexpr int kTiledMinRows = 129;
// From this many rows (five 256-row tiles, 160 workgroups of 256 x 256 on
// 256 CUs) the expert's gate/up uses the square-tile GEMM.
constexpr int kSqMinRows = 1025;

// L2 warm-up of a later kernel's operands by spare workgroups appended to a
// launch.  A workgroup's XCD (and so its L2) follows its linear block index
// mod 8 with one fixed offset for every kernel, so a prefetching workgroup
// whose index matches a consumer workgroup's mod 8 fills the consumer's L2.
//   slices: the consumer's workgroup j reads bytes [j*bytes, (j+1)*bytes) of
//           base, j < count;
//   broadcast (count == 0): every XCD's L2 gets all `bytes` of base.
struct Prefetch {
  const void* base;
  uint32_t bytes;
  int count;
};
struct PrefetchSet {
  Prefetch r[3];
  int nwg;        // columns of prefetching workgroups appended (multiple of 8; 0 = none)
};

struct IoParams {
  PrefetchSet pf;
  const DevArgs* da;
  float* h;               // [Mpad][1024] fp32 residual stream
  const uint16_t* w_in;   // action_in W [1024][32] bf16
  const float* b_in;      // [1024]
  const uint16_t* w_out;  // action_out W [32][1024] bf16
  const float* fin_s1;    // final (1+scale) for the finishing step [1024] (null: no final norm)
  const float* c_out;     // [32] shift @ W_out^T + b_out for the finishing step
  const float* s1_next;   // (1 + scale) of the first layer's attention norm (do_in)
  uint16_t* u_out;        // its operand bf16(h * (1 + scale)), fragment-major
  float* ssq_out;         // partial sums of h^2 [Mpad][64]
  float dt;
  float eps;
  int do_out;             // finish the previous step: final norm, out proj, Euler
  int do_in;              // start a step: action_in
  int from_noise;         // x comes from noise (first step)
  int M;
  // pi0 action-time encoder (enc = 1): do_in computes z = SiLU(x W_in^T + b_in)
  // (W_in, b_in: the folded encoder input and this step's bias) into u_out as
  // the operand of the encoder's output GEMM [Mpad/16][32][64][8], and sets
  // h = h_init (that GEMM's bias, to which it adds); no u / h^2 partials
  const float* h_init;
  int enc;
};

struct GemmParams {
  PrefetchSet pf;
  const uint16_t* w;      // swizzled weight fragments of this layer
  int M;                  // valid rows
  // A operand: bf16 fragment-major [Mpad/16][K/32][64][8]
  const uint16_t* a_frag; // u (QKV, GU), O or m
  const float* ssq;       // QKV, GU: per-row partial sums of h^2 [Mpad][64]
  float eps;
  // epilogue
  const float* bias;      // QKV / GU: shift-fold bias in the swizzled column order
  const float* gate;      // residual modes: per-column gate [1024]
  float* h_out;           // residual modes: fp32 residual stream
  const float* s1_next;   // residual modes: (1 + scale) of the next normalised GEMM, or null
  uint16_t* u_out;        //   its operand bf16(h * (1 + scale)), fragment-major [Mpad/16][32][64][8]
  float* ssq_out;         //   and the partial sums of h^2 [Mpad][64]
  uint16_t* q_out;        // QKV: Q [M][8][256]
  const float2* rope_cs;  // QKV: (cos, sin) of each suffix row's position [M][128]
  int T;                  // chunk length (rows per episode)
  int P, nkb;             // prefix length, 32-key blocks per episode of the packed K/V
  uint16_t* kp;           // QKV: packed K of this layer (suffix keys written here)
  uint16_t* vp;           // QKV: packed V of this layer
  uint16_t* m_out;        // GU: m, fragment-major [Mpad/16][128][64][8]
  // O with the attention split over two key ranges (small M): a_frag and
  // a_frag2 hold the two normalised partial outputs, astat [M][8][4] each
  // query row's (max, sum) of both; the A operand is their weighted mean
  const uint16_t* a_frag2;
  const float* astat;
  // QKV of the VLM prefill: this layer's K (rotated) and V in natural layout
  // [M][256], the cache the expert reads (null: not written)
  uint16_t* k_cache;
  uint16_t* v_cache;
  // vision epilogues: the position embedding [256][1152] fp32 (patch
  // embedding); their natural bf16 outputs go to q_out (Q|K|V [M][3456],
  // projector [M][2048]), the MLP operand to m_out, the residual to h_out
  const float* aux;
};

struct AttnParams {
  PrefetchSet pf;
  const uint16_t* q;      // [M][8][256]
  const uint16_t* kp;     // packed K of this layer [B][nkb][16][64][8]
  const uint16_t* vp;     // packed V of this layer [B][nkb][16][64][8]
  const float* kbias;     // [B][nkb*32]: 0 valid, -inf masked / padding
  uint16_t* o;            // fragment-major [Mpad/16][64][64][8]
  // o2 != null: each query block's keys are split over two workgroups; key
  // range s writes its normalised partial output to (s ? o2 : o) and its
  // (max, sum) to the row statistics fp32 [M * 8][4] (elements 2s, 2s+1),
  // which follow the second output: attn_row_stats(o2, B * T).
  // (Kept at 120 bytes: a larger argument block measurably slows this kernel.)
  uint16_t* o2;
  int B, T, P, nkb;
};
// Where the attention row statistics live: right after the second partial
// output, whose fragment-major rows are padded to a multiple of 16.
inline __host__ __device__ float* attn_row_stats(uint16_t* o2, int M) {
  return reinterpret_cast<float*>(o2 + size_t((M + 15) / 16) * 16 * kH * kHd);
}

struct PackParams {
  const DevArgs* da;
  const int* n_valid;     // [B]
  const double* inv_freq; // RoPE inverse frequencies base^(-2i/256) [128]
  float2* rope_cs;        // out: (cos, sin) of each suffix row's position [B*T][128]
  uint16_t* kp;           // [L][B][nkb][16][64][8]
  uint16_t* vp;
  float* kbias;           // [B][nkb*32]
  int B, P, T, nkb;
};

// Staging of one VLM prefill call (one workgroup per prefix row): the residual
// stream h = the prefix sequence, the first layer's operand bf16(h * gamma)
// with its h^2 partials, each row's RoPE (cos, sin) at its position (the number
// of valid tokens before it in its episode) and the additive key bias of the
// episode's keys.
struct VlmStageParams {
  const uint16_t* emb;    // [B][P][2048] bf16, the scaled prefix sequence
  const uint8_t* mask;    // [B][P] or null (all valid)
  const float* s1;        // the first layer's attention-norm scale [2048]
  const double* inv_freq; // RoPE inverse frequencies [128]
  float* h;               // [Mpad][2048]
  uint16_t* u;            // fragment-major [Mpad/16][64][64][8]
  float* ssq;             // [Mpad][128]
  float2* rope_cs;        // [B*P][128]
  float* kbias;           // [B][nkb*32]
  int B, P, nkb;
};

// Vision encoder, per call: the patch vectors of every view (im2col of the
// 14x14x3 patches, (channel, y, x) order, zero-padded to 768) as the patch
// GEMM's fragment-major operand.
struct VisPatchParams {
  const uint16_t* images;  // [V][224][224][3] bf16
  uint16_t* a;             // fragment-major [Mpad/16][768/32][64][8]
  int V;
};
// LayerNorm of the residual stream into a GEMM operand: u = (h - mean) /
// sqrt(var + eps) * w + b, bf16, fragment-major [Mpad/16][1280/32][64][8]
// (columns 1152.. stay zero).
struct VisLnParams {
  float* h;                // [Mpad][1152]
  const float* w;          // [1152]
  const float* b;          // [1152]
  uint16_t* u;
  float eps;
  int M;
  // residual form (launch_vis_res_ln): first h += sum of the S partial tiles
  // part[z][Mp][1152] of a 1152-column GEMM (fixed order z = 0 .. S-1) +
  // bias, then the LayerNorm of the new h
  const float* part;
  const float* bias;       // [1152]
  int S, Mp;
};
// Attention of one view's 256 tokens, 16 heads x 72, all keys valid.
struct VisAttnParams {
  const uint16_t* qkv;     // [M][3456] natural: q | k | v, head h at columns 72h..
  uint16_t* o;             // fragment-major [Mpad/16][1280/32][64][8]
  int V;
};

struct ArgsParams {
  DevArgs* da;
  DevArgs vals;
  int* n_valid;
  int B, P;
};

// Optional per-launch timing: events recorded at the kernel's own start and
// end (used to time one kernel inside the real loop).
struct KernelTiming {
  hipEvent_t start, stop;
};

hipError_t launch_args(const ArgsParams& p, hipStream_t s);
hipError_t launch_io(const IoParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_qkv(const GemmParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_attn(const AttnParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_pack(const PackParams& p, int L, hipStream_t s);
hipError_t launch_o(const GemmParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_gu(const GemmParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_down(const GemmParams& p, hipStream_t s, const KernelTiming* t = nullptr);
// h += acc * gate with K = 1024 (the pi0 encoder's output layer), the same
// residual epilogue as O and down
hipError_t launch_enc(const GemmParams& p, hipStream_t s);

// VLM prefill (width 2048, MLP 16384; always the tiled GEMMs)
hipError_t launch_vlm_stage(const VlmStageParams& p, hipStream_t s);
// kv_only: the K/V columns only (the last layer).  S > 1 splits K over S
// workgroups per tile (K / S a multiple of 256) with fp32 partials in `part`
// (S x row_tiles(M, 128) * 128 x N floats), summed by a second kernel that
// runs the epilogue.
hipError_t launch_vlm_qkv(const GemmParams& p, bool kv_only, int S, float* part, hipStream_t s,
                          const KernelTiming* t = nullptr);
hipError_t launch_vlm_attn(const AttnParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_vlm_o(const GemmParams& p, int S, float* part, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_vlm_gu(const GemmParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_vlm_down(const GemmParams& p, int S, float* part, hipStream_t s, const KernelTiming* t = nullptr);

// vision encoder (tiled GEMMs with the vision epilogues; which: 0 patch
// embedding, 1 QKV, 2 O + residual, 3 fc1 + GELU, 4 fc2 + residual, 5
// projector).  S > 1 splits K (fc2 only).
hipError_t launch_vis_patch(const VisPatchParams& p, hipStream_t s);
hipError_t launch_vis_ln(const VisLnParams& p, hipStream_t s);
hipError_t launch_vis_res_ln(const VisLnParams& p, hipStream_t s, const KernelTiming* t = nullptr);
// which as in launch_vis_gemm (2 = O, 4 = fc2): only the raw K-split GEMM
// (S ranges into part[z][Mp][1152]); launch_vis_res_ln finishes it
hipError_t launch_vis_gemm_raw(int which, const GemmParams& p, int S, float* part, hipStream_t s,
                               const KernelTiming* t = nullptr);
hipError_t launch_vis_attn(const VisAttnParams& p, hipStream_t s, const KernelTiming* t = nullptr);
hipError_t launch_vis_gemm(int which, const GemmParams& p, int S, float* part, hipStream_t s,
                           const KernelTiming* t = nullptr);

// The fixed device array of the allocation-free entry point (one copy per GPU,
// defined in pi_ae_noalloc.hip): its capacity, the largest number of GEMM rows
// a call through it may have (the weight-streaming kernels' row range), and
// the lookup of its device address on the current GPU (once per device).
constexpr size_t kNoallocScratchBytes = size_t(24) << 20;
constexpr int kNoallocMaxRows = 64;
hipError_t noalloc_scratch(void** ptr);

// The thread-local message that pi_ae_last_error returns (set by every
// translation unit of the library on failure).
void set_last_error(const std::string& msg);

// Swizzled weight geometry (shared by prep and kernels): a weight W[N][K]
// (nn.Linear layout) is stored as 1 KiB fragments, fragment (nb, kb) =
// columns n in [16nb, 16nb+16), k in [32kb, 32kb+32); lane l of the fragment
// holds W[16nb + l%16][32kb + 8(l/16) .. +8] (the B operand of
// v_mfma_f32_16x16x32_bf16), fragments ordered nb-major.
inline size_t frag_offset(int nb, int kb, int KB) { return (size_t(nb) * KB + kb) * 512; }

}  // namespace pi_ae
