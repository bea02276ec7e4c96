// gfx950 (CDNA4) kernels of the action-expert flow-matching denoise loop.
//
// One denoise step (Realtime-VLA technical blog, section "pi0.5 inference
// flow"; per-layer list in section "LeRobot implementation") is, per expert
// layer:  QKV + RoPE  ->  attention over prefix + suffix keys  ->  O projection
// with gated residual  ->  gate/up with GELU(gate) * up  ->  down projection
// with gated residual;  plus a row-local kernel between steps (final norm,
// action_out_proj, Euler update, next step's action_in_proj).
//
// Batch-1 steps stream ~623 MB of bf16 weights for 63 tokens, so the GEMMs
// here are weight-streaming kernels: every wave issues all of its weight
// fragment loads (pre-swizzled into the MFMA B-operand lane order, 1 KiB per
// 16x32 fragment, fully coalesced) before touching activations, the waves of
// a workgroup split K, and the split-K partials are reduced through LDS where
// the fused epilogue runs.  Activations stay L2-resident between kernels.
#include "pi_ae_kernels.h"

#include <math.h>

namespace pi_ae {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ bf16x8 as_bf(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 pack8(float4 lo, float4 hi) {
  f32x8 v = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// GELU, tanh approximation (the MLP activation of the Gemma-shaped expert).
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c = 0.7978845608028654f;
  return 0.5f * x * (1.f + tanhf(c * (x + 0.044715f * x * x * x)));
}
// Offset (in bf16 elements) of activation (row, k) in the fragment-major
// layout [rows/16][K/32][64 lanes][8] that the GEMM A operand loads directly.
__device__ __forceinline__ size_t afrag_index(int row, int k, int KB) {
  const int lane = (row & 15) + 16 * ((k & 31) >> 3);
  return ((size_t(row >> 4) * KB + (k >> 5)) * 64 + lane) * 8 + (k & 7);
}

// Packed per-layer K/V of one call, 32-key blocks of 16 KiB per episode:
//   K: [b][key/32][mk = (key%32)/16][ks = d/32][lane][8] with lane = key%16 +
//      16 ((d%32)/8): the A operand of S^T = K Q^T, one 1 KiB fragment per (mk, ks);
//   V: [b][key/32][md = d/16][lane][8] with lane = d%16 + 16 g, where the 8
//      values of group g are keys 4g..4g+3 and 16+4g..16+4g+3 of the block: the
//      A operand of O^T = V^T P^T in the key order the probabilities sit in.
__device__ __forceinline__ size_t kpack_index(int b, int key, int d, int nkb) {
  const int w32 = key & 31;
  const int lane = (w32 & 15) + 16 * ((d & 31) >> 3);
  return ((size_t(b) * nkb + (key >> 5)) * 16 + (w32 >> 4) * 8 + (d >> 5)) * 512 + lane * 8 + (d & 7);
}
__device__ __forceinline__ size_t vpack_index(int b, int key, int d, int nkb) {
  const int kk = key & 31, r4 = kk & 15;
  const int lane = (d & 15) + 16 * (r4 >> 2);
  return ((size_t(b) * nkb + (key >> 5)) * 16 + (d >> 4)) * 512 + lane * 8 + (kk >> 4) * 4 + (r4 & 3);
}

// ---------------------------------------------------------------------------
// Per-call staging: publish the call's pointers to the graph and count each
// episode's valid prefix keys (the suffix RoPE positions start there; the
// blog's prefix/suffix softmax kernel likewise reads the prefix valid length
// dynamically).
__global__ __launch_bounds__(256) void k_args(ArgsParams p) {
  __shared__ int cnt;
  if (threadIdx.x == 0) *p.da = p.vals;
  for (int b = 0; b < p.B; ++b) {
    if (threadIdx.x == 0) cnt = 0;
    __syncthreads();
    int c = 0;
    if (p.vals.mask) {
      const uint8_t* mrow = p.vals.mask + size_t(b) * p.P;
      for (int i = threadIdx.x; i < p.P; i += blockDim.x) c += mrow[i] != 0;
    } else if (threadIdx.x == 0) {
      c = p.P;
    }
    if (c) atomicAdd(&cnt, c);
    __syncthreads();
    if (threadIdx.x == 0) p.n_valid[b] = cnt;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Step boundary, one workgroup per token row:
//   do_out: final AdaRMS norm (scale only; the shift is folded into c_out),
//           v = u W_out^T + c_out, Euler x <- x + dt v   (the blog's "pi0.5
//           inference flow", steps 3-4; dt applied in fp32);
//   do_in:  h = x W_in^T + b_in                          (action_in_proj).
__global__ __launch_bounds__(256) void k_io(IoParams p) {
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  __shared__ float su[kD];
  __shared__ float sred[4];
  __shared__ float sx[kA];
  float* x = p.da->actions + size_t(row) * kA;
  if (t < kA) sx[t] = p.from_noise ? p.da->noise[size_t(row) * kA + t] : x[t];
  if (p.do_out) {
    float4 hv = reinterpret_cast<const float4*>(p.h + size_t(row) * kD)[t];
    if (p.fin_s1) {
      float ss = wave_sum(hv.x * hv.x + hv.y * hv.y + hv.z * hv.z + hv.w * hv.w);
      if (lane == 0) sred[w] = ss;
      __syncthreads();
      const float r = 1.f / sqrtf((sred[0] + sred[1] + sred[2] + sred[3]) * (1.f / kD) + p.eps);
      const float4 s = reinterpret_cast<const float4*>(p.fin_s1)[t];
      hv = make_float4(hv.x * r * s.x, hv.y * r * s.y, hv.z * r * s.z, hv.w * r * s.w);
    }
    reinterpret_cast<float4*>(su)[t] = hv;
    __syncthreads();
    // wave w: outputs 8w..8w+7; lane covers input columns 16*lane .. +16
    float part[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const uint4* wr = reinterpret_cast<const uint4*>(p.w_out + size_t(8 * w + a) * kD + 16 * lane);
      const uint4 w0 = wr[0], w1 = wr[1];
      const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        acc += su[16 * lane + 2 * q] * bf2f(ww[q] & 0xffffu);
        acc += su[16 * lane + 2 * q + 1] * bf2f(ww[q] >> 16);
      }
      part[a] = wave_sum(acc);
    }
    if (lane == 0) {
#pragma unroll
      for (int a = 0; a < 8; ++a) sx[8 * w + a] += p.dt * (part[a] + p.c_out[8 * w + a]);
    }
  }
  __syncthreads();
  if (p.do_in) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = 4 * t + q;
      const uint4* wr = reinterpret_cast<const uint4*>(p.w_in + size_t(n) * kA);
      float acc = p.b_in[n];
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const uint4 wv = wr[v4];
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += sx[8 * v4 + 2 * e] * bf2f(ww[e] & 0xffffu);
          acc += sx[8 * v4 + 2 * e + 1] * bf2f(ww[e] >> 16);
        }
      }
      su[n] = acc;
    }
    // (su is free here: every read of it above happened before the barrier)
    __syncthreads();
    reinterpret_cast<float4*>(p.h + size_t(row) * kD)[t] = reinterpret_cast<const float4*>(su)[t];
  }
  if (t < kA) x[t] = sx[t];
}

// ---------------------------------------------------------------------------
// Weight-streaming GEMM.  Workgroup tile: MB*16 rows x NB*16 columns, NW
// waves each owning KBW consecutive 32-wide K blocks (intra-workgroup split-K).
//   A_NORM: A = bf16(h * (1 + scale)) built from the fp32 residual stream; the
//           RMS statistics of the full rows are reduced across the waves and
//           1/rms is applied in the epilogue (it commutes with the GEMM).
//   A_FRAG: A = bf16 activations stored fragment-major by their producer.
// Epilogues:
//   E_QKV:  + shift-fold bias, RoPE on (i, i+128) pairs, scatter Q/K_s/V_s.
//   E_GELU: + shift-fold bias, m = GELU(gate) * up, store m fragment-major.
//   E_RES:  h += acc * gate (gated residual).
enum { A_NORM = 0, A_FRAG = 1 };
enum { E_QKV = 0, E_GELU = 1, E_RES = 2 };

template <int MB, int NB, int NW, int KBW, int AMODE, int EPI>
__global__ __launch_bounds__(NW * 64) void k_gemm(GemmParams p) {
  constexpr int KB = KBW * NW;
  constexpr int E = MB * NB * 4 * 64;  // accumulator floats per wave
  constexpr int NT = NW * 64;
  static_assert(AMODE != A_NORM || KB * 32 == kD, "normalised input spans the full width");
  static_assert(EPI == E_RES || NB == 2, "paired epilogues take two n-blocks");
  __shared__ float red[NW * E];
  __shared__ float ssq[NW * MB * 16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int j = blockIdx.x;
  const int row0 = blockIdx.y * MB * 16;

  // 1. this wave's weight fragments, all in flight before any activation load
  uint4 bw[NB][KBW];
  const uint4* wp = reinterpret_cast<const uint4*>(p.w);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
      bw[nb][kb] = wp[(size_t(j * NB + nb) * KB + w * KBW + kb) * 64 + lane];

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ss[mb] = 0.f;

  // 2. K loop over this wave's blocks.  Activation loads run PF blocks ahead
  // of the MFMAs; scheduling barriers keep every weight load ahead of the
  // first wait (vmcnt retires loads in issue order).
  constexpr int PF = KBW < 4 ? KBW : 4;
  constexpr int AW = (AMODE == A_NORM) ? 2 : 1;  // 16-byte loads per (row block, K block)
  uint4 abuf[PF][MB][AW];
  float4 sbuf[PF][AW];
  const uint4* ap = reinterpret_cast<const uint4*>(p.a_frag);
#define PI_AE_LOAD_A(KBI, SLOT)                                                                  \
  {                                                                                              \
    if constexpr (AMODE == A_NORM) {                                                             \
      const int k_ = (w * KBW + (KBI)) * 32 + 8 * g;                                             \
      sbuf[SLOT][0] = *reinterpret_cast<const float4*>(p.s1 + k_);                               \
      sbuf[SLOT][AW - 1] = *reinterpret_cast<const float4*>(p.s1 + k_ + 4);                      \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                        \
        const int row_ = row0 + mb * 16 + c;                                                     \
        const uint4* hp_ = reinterpret_cast<const uint4*>(p.h + size_t(row_ < p.M ? row_ : 0) * kD + k_); \
        abuf[SLOT][mb][0] = hp_[0];                                                              \
        abuf[SLOT][mb][AW - 1] = hp_[1];                                                         \
      }                                                                                          \
    } else {                                                                                     \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                          \
        abuf[SLOT][mb][0] = ap[(size_t((row0 >> 4) + mb) * KB + w * KBW + (KBI)) * 64 + lane];    \
    }                                                                                            \
  }
#pragma unroll
  for (int kb = 0; kb < PF; ++kb) PI_AE_LOAD_A(kb, kb)

  // epilogue operands that do not depend on the GEMM, in flight during it
  constexpr int EPT = (EPI == E_RES) ? E / NT : 1;        // residual elements per thread
  constexpr int PPT = (EPI == E_RES) ? 1 : MB * 256 / NT;  // output pairs per thread
  static_assert(E % NT == 0 && (MB * 256) % NT == 0, "epilogue work divides evenly");
  float eh[EPT], eg[EPT];
  float eb0[PPT], eb1[PPT], einv[PPT];
  int env[PPT];
  if constexpr (EPI == E_RES) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = threadIdx.x + q * NT;
      const int mb = e / (NB * 256), nb = (e >> 8) % NB, i = (e >> 6) & 3, ln = e & 63;
      const int row = row0 + mb * 16 + 4 * (ln >> 4) + i;
      const int col = (j * NB + nb) * 16 + (ln & 15);
      eh[q] = p.h_out[size_t(row < p.M ? row : 0) * kD + col];
      eg[q] = p.gate[col];
    }
  } else {
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int pi = threadIdx.x + q * NT;
      const int i = (pi >> 6) & 3, ln = pi & 63, mb = pi >> 8;
      const int cc = ln & 15, rl = mb * 16 + 4 * (ln >> 4) + i, row = row0 + rl;
      eb0[q] = p.bias[(2 * j) * 16 + cc];
      eb1[q] = p.bias[(2 * j + 1) * 16 + cc];
      if constexpr (EPI == E_QKV) {
        einv[q] = p.inv_freq[(j & 7) * 16 + cc];
        env[q] = p.n_valid[(row < p.M ? row : 0) / p.T];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    const int slot = kb % PF;
    bf16x8 af[MB];
    if constexpr (AMODE == A_NORM) {
      const float4 s0 = sbuf[slot][0], s1 = sbuf[slot][AW - 1];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bool live = row0 + mb * 16 + c < p.M;
        float4 lo = __builtin_bit_cast(float4, abuf[slot][mb][0]);
        float4 hi = __builtin_bit_cast(float4, abuf[slot][mb][AW - 1]);
        if (!live) lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
        ss[mb] += lo.x * lo.x + lo.y * lo.y + lo.z * lo.z + lo.w * lo.w + hi.x * hi.x + hi.y * hi.y + hi.z * hi.z +
                  hi.w * hi.w;
        af[mb] = pack8(make_float4(lo.x * s0.x, lo.y * s0.y, lo.z * s0.z, lo.w * s0.w),
                       make_float4(hi.x * s1.x, hi.y * s1.y, hi.z * s1.z, hi.w * s1.w));
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = as_bf(abuf[slot][mb][0]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma(af[mb], as_bf(bw[nb][kb]), acc[mb][nb]);
    if (kb + PF < KBW) PI_AE_LOAD_A(kb + PF, slot)
    __builtin_amdgcn_sched_barrier(0);
  }
#undef PI_AE_LOAD_A

  // 3. split-K partials (and row statistics) through LDS
  if constexpr (AMODE == A_NORM) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      ss[mb] += __shfl_xor(ss[mb], 16);
      ss[mb] += __shfl_xor(ss[mb], 32);
    }
    if (lane < 16) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) ssq[w * MB * 16 + mb * 16 + lane] = ss[mb];
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w * E + ((mb * NB + nb) * 4 + i) * 64 + lane] = acc[mb][nb][i];
  __syncthreads();

  auto rstd = [&](int rl) {
    float s = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) s += ssq[w2 * MB * 16 + rl];
    return 1.f / sqrtf(s * (1.f / kD) + p.eps);
  };

  if constexpr (EPI == E_RES) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = threadIdx.x + q * NT;
      float x = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) x += red[w2 * E + e];
      const int mb = e / (NB * 256), nb = (e >> 8) % NB, i = (e >> 6) & 3, ln = e & 63;
      const int row = row0 + mb * 16 + 4 * (ln >> 4) + i;
      const int col = (j * NB + nb) * 16 + (ln & 15);
      if (row < p.M) p.h_out[size_t(row) * kD + col] = eh[q] + x * eg[q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < PPT; ++q) {
      const int pi = threadIdx.x + q * NT;
      const int mb = pi >> 8, i = (pi >> 6) & 3, ln = pi & 63;
      const int e0 = ((mb * 2 + 0) * 4 + i) * 64 + ln, e1 = ((mb * 2 + 1) * 4 + i) * 64 + ln;
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        x0 += red[w2 * E + e0];
        x1 += red[w2 * E + e1];
      }
      const int rl = mb * 16 + 4 * (ln >> 4) + i, cc = ln & 15;
      const int row = row0 + rl;
      if (row >= p.M) continue;
      const float r = rstd(rl);
      const float y0 = x0 * r + eb0[q];
      const float y1 = x1 * r + eb1[q];
      if constexpr (EPI == E_QKV) {
        const int b = row / p.T, t = row - b * p.T;
        if (j < 72) {  // Q heads (j < 64) and K_s (64 <= j < 72): rotate pair (ip, ip+128)
          const int ip = (j & 7) * 16 + cc;
          float sn, cs;
          sincosf(float(env[q] + t) * einv[q], &sn, &cs);
          const float o0 = y0 * cs - y1 * sn;
          const float o1 = y1 * cs + y0 * sn;
          if (j < 64) {
            uint16_t* dst = p.q_out + (size_t(row) * kH + (j >> 3)) * kHd;
            dst[ip] = f2bf(o0);
            dst[kRopeHalf + ip] = f2bf(o1);
          } else {
            const int key = p.P + t;
            p.kp[kpack_index(b, key, ip, p.nkb)] = f2bf(o0);
            p.kp[kpack_index(b, key, kRopeHalf + ip, p.nkb)] = f2bf(o1);
          }
        } else {  // V_s: no rotation
          const int key = p.P + t, d0 = (j - 72) * 32 + cc;
          p.vp[vpack_index(b, key, d0, p.nkb)] = f2bf(y0);
          p.vp[vpack_index(b, key, d0 + 16, p.nkb)] = f2bf(y1);
        }
      } else {  // E_GELU: n-block 0 = gate columns 16j.., n-block 1 = the same up columns
        const int f = 16 * j + cc;
        p.m_out[afrag_index(row, f, kF / 32)] = f2bf(gelu_tanh(y0) * y1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per call, once: pack every layer's prefix K/V into the attention's operand
// order (see kpack_index / vpack_index) and build the additive key bias of
// each episode: 0 for valid prefix keys and for the suffix keys, -inf for
// pad-masked prefix keys and block padding (the blog's prefix/suffix softmax
// kernel fills invalid keys with -2.38e38; -inf gives the same exp = 0).
// Masked and padding keys are stored as zeros so that garbage in the cache
// cannot reach the result.  Suffix keys are written later by the QKV kernel.
// grid (nkb, B, L), 256 threads; each workgroup packs one 32-key block.
__global__ __launch_bounds__(256) void k_pack(PackParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t vs[32][kHd + 8];
  const int kb = blockIdx.x, b = blockIdx.y, l = blockIdx.z, t = threadIdx.x;
  const DevArgs* da = p.da;
  const size_t lay = size_t(l) * p.B * p.P * kHd;
  const uint16_t* pk = da->pk + lay + size_t(b) * p.P * kHd;
  const uint16_t* pv = da->pv + lay + size_t(b) * p.P * kHd;
  const uint8_t* mask = da->mask ? da->mask + size_t(b) * p.P : nullptr;
  uint16_t* kp = p.kp + (size_t(l) * p.B + b) * p.nkb * 8192 + size_t(kb) * 8192;
  uint16_t* vp = p.vp + (size_t(l) * p.B + b) * p.nkb * 8192 + size_t(kb) * 8192;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  // K: 1024 16-byte chunks per block, each a straight copy of part of one key row
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int chunk = t + 256 * q;         // (mk*8 + ks)*64 + lane
    const int lane = chunk & 63, f = chunk >> 6, mk = f >> 3, ks = f & 7;
    const int key = kb * 32 + mk * 16 + (lane & 15);
    const bool ok = key < p.P && (!mask || mask[key] != 0);
    reinterpret_cast<uint4*>(kp)[chunk] =
        ok ? *reinterpret_cast<const uint4*>(pk + size_t(key) * kHd + ks * 32 + 8 * (lane >> 4)) : zero4;
  }
  // V: stage the 32 key rows, then gather 8 keys per 16-byte chunk
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int chunk = t + 256 * q;         // key row kk, 16-byte column dc
    const int kk = chunk >> 5, dc = chunk & 31, key = kb * 32 + kk;
    const bool ok = key < p.P && (!mask || mask[key] != 0);
    *reinterpret_cast<uint4*>(&vs[kk][dc * 8]) =
        ok ? *reinterpret_cast<const uint4*>(pv + size_t(key) * kHd + dc * 8) : zero4;
  }
  __syncthreads();
  if (kb * 32 < p.P) {  // blocks made only of suffix keys / padding are written by the QKV kernel / stay zero
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int chunk = t + 256 * q;       // md*64 + lane
      const int lane = chunk & 63, md = chunk >> 6, d = md * 16 + (lane & 15), g = lane >> 4;
      uint16_t e[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) e[jj] = vs[(jj < 4) ? 4 * g + jj : 16 + 4 * g + (jj - 4)][d];
      uint4 o;
      o.x = e[0] | (uint32_t(e[1]) << 16);
      o.y = e[2] | (uint32_t(e[3]) << 16);
      o.z = e[4] | (uint32_t(e[5]) << 16);
      o.w = e[6] | (uint32_t(e[7]) << 16);
      reinterpret_cast<uint4*>(vp)[chunk] = o;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) reinterpret_cast<uint4*>(vp)[t + 256 * q] = zero4;
  }
  if (l == 0 && t < 32) {
    const int key = kb * 32 + t;
    const bool ok = key < p.P ? (!mask || mask[key] != 0) : key < p.P + p.T;
    p.kbias[size_t(b) * p.nkb * 32 + key] = ok ? 0.f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Attention of 8 query heads sharing one KV head over the episode's prefix
// keys (read-only cache, pad-masked) and all of its suffix keys ("LeRobot
// implementation": repeat_kv -> Q K^T * scaling -> softmax -> V).  Queries are
// the episode's (token, head) rows, so every query sees the same key set and
// one K/V stream serves all heads.  Workgroup: 16 queries; its 4 waves split
// the 32-key blocks (online softmax in fp32) and are merged through LDS.
// Scores are computed transposed (S^T = K Q^T) so that the probabilities land
// in the B-operand lane order of O^T = V^T P^T; K and V arrive packed in
// operand order, so every load is one contiguous 1 KiB fragment per wave, and
// the next block's K is in flight while the current block is processed.
constexpr int kOStride = 260;  // floats per query row in the merge buffer

__global__ __launch_bounds__(256) void k_attn(AttnParams p) {
  __shared__ __attribute__((aligned(16))) float ored[4 * 16 * kOStride + 4 * 16 * 2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.y;
  const int nq = p.T * kH;
  const int r = blockIdx.x * 16 + c;
  const int rc = r < nq ? r : nq - 1;

  bf16x8 qf[8];
  const uint16_t* qrow = p.q + (size_t(b) * nq + rc) * kHd;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf(*reinterpret_cast<const uint4*>(qrow + ks * 32 + 8 * g));

  const int nkb = p.nkb;
  const int kb0 = w * nkb / 4, kb1 = (w + 1) * nkb / 4;
  const uint4* kp = reinterpret_cast<const uint4*>(p.kp) + size_t(b) * nkb * 1024;
  const uint4* vp = reinterpret_cast<const uint4*>(p.vp) + size_t(b) * nkb * 1024;
  const float* kbias = p.kbias + size_t(b) * nkb * 32;

  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = 0.0625f * 1.4426950408889634f;  // 1/sqrt(256) * log2(e)

  uint4 kf[16];
  if (kb0 < kb1) {
#pragma unroll
    for (int f = 0; f < 16; ++f) kf[f] = kp[size_t(kb0) * 1024 + f * 64 + lane];
  }
  for (int kb = kb0; kb < kb1; ++kb) {
    uint4 vf[16];
#pragma unroll
    for (int md = 0; md < 16; ++md) vf[md] = vp[size_t(kb) * 1024 + md * 64 + lane];
    const float4 bl = *reinterpret_cast<const float4*>(kbias + kb * 32 + 4 * g);
    const float4 bh = *reinterpret_cast<const float4*>(kbias + kb * 32 + 16 + 4 * g);
    // scores S^T[key][query] for the 32 keys of this block
    f32x4 s[2];
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
      s[mk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s[mk] = mfma(as_bf(kf[mk * 8 + ks]), qf[ks], s[mk]);
    }
    if (kb + 1 < kb1) {
#pragma unroll
      for (int f = 0; f < 16; ++f) kf[f] = kp[size_t(kb + 1) * 1024 + f * 64 + lane];
    }
    const float bias[2][4] = {{bl.x, bl.y, bl.z, bl.w}, {bh.x, bh.y, bh.z, bh.w}};
    float pr[2][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int mk = 0; mk < 2; ++mk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[mk][i] = s[mk][i] * sc + bias[mk][i];
        mloc = fmaxf(mloc, pr[mk][i]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const bool none = (m_new == -INFINITY);
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int mk = 0; mk < 2; ++mk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[mk][i] = none ? 0.f : exp2f(pr[mk][i] - m_new);
        lsum += pr[mk][i];
      }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    const bf16x8 pf = pack8(make_float4(pr[0][0], pr[0][1], pr[0][2], pr[0][3]),
                            make_float4(pr[1][0], pr[1][1], pr[1][2], pr[1][3]));
#pragma unroll
    for (int md = 0; md < 16; ++md) acc[md] = mfma(as_bf(vf[md]), pf, acc[md] * alpha);
  }

  // merge the 4 key ranges
  float* sml = ored + 4 * 16 * kOStride;  // [4][16][2]
#pragma unroll
  for (int md = 0; md < 16; ++md)
#pragma unroll
    for (int i = 0; i < 4; ++i) ored[(w * 16 + c) * kOStride + md * 16 + 4 * g + i] = acc[md][i];
  if (g == 0) {
    sml[(w * 16 + c) * 2] = m_run;
    sml[(w * 16 + c) * 2 + 1] = l_run;
  }
  __syncthreads();
  const int q = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 16;
  float mw[4], f[4];
  float mmax = -INFINITY;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    mw[w2] = sml[(w2 * 16 + q) * 2];
    mmax = fmaxf(mmax, mw[w2]);
  }
  float L = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    f[w2] = (mw[w2] == -INFINITY) ? 0.f : exp2f(mw[w2] - mmax);
    L += f[w2] * sml[(w2 * 16 + q) * 2 + 1];
  }
  const float inv = 1.f / L;
  const int rq = blockIdx.x * 16 + q;
  if (rq < nq) {
    const int trow = b * p.T + rq / kH, head = rq % kH;
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) sum += f[w2] * ored[(w2 * 16 + q) * kOStride + d0 + 8 * h8 + e];
        o[e] = sum * inv;
      }
      const uint4 packed = __builtin_bit_cast(uint4, pack8(make_float4(o[0], o[1], o[2], o[3]),
                                                            make_float4(o[4], o[5], o[6], o[7])));
      *reinterpret_cast<uint4*>(p.o + afrag_index(trow, head * kHd + d0 + 8 * h8, (kH * kHd) / 32)) = packed;
    }
  }
}

// ---------------------------------------------------------------------------
static inline unsigned row_tiles(int M) { return unsigned((M + 63) / 64); }

hipError_t launch_args(const ArgsParams& p, hipStream_t s) {
  k_args<<<1, 256, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_io(const IoParams& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  k_io<<<p.M, 256, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_qkv(const GemmParams& p, hipStream_t s) {
  k_gemm<4, 2, 4, 8, A_NORM, E_QKV><<<dim3(kNqkv / 32, row_tiles(p.M)), 256, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_gu(const GemmParams& p, hipStream_t s) {
  k_gemm<4, 2, 4, 8, A_NORM, E_GELU><<<dim3(kNgu / 32, row_tiles(p.M)), 256, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_o(const GemmParams& p, hipStream_t s) {
  k_gemm<4, 1, 8, 8, A_FRAG, E_RES><<<dim3(kD / 16, row_tiles(p.M)), 512, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_down(const GemmParams& p, hipStream_t s) {
  k_gemm<4, 1, 8, 16, A_FRAG, E_RES><<<dim3(kD / 16, row_tiles(p.M)), 512, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  k_attn<<<dim3((p.T * kH + 15) / 16, p.B), 256, 0, s>>>(p);
  return hipGetLastError();
}
hipError_t launch_pack(const PackParams& p, int L, hipStream_t s) {
  if (p.B <= 0 || p.nkb <= 0) return hipSuccess;
  k_pack<<<dim3(p.nkb, p.B, L), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace pi_ae
