// Host runtime of libpi_ae.so: argument validation, one-time weight
// preparation (fp64 tabulation and folding, fused and swizzled weights),
// workspaces, the per-(batch, prefix) hipGraph cache and the C ABI.
#include "pi_ae.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "pi_ae_kernels.h"

using namespace pi_ae;

#define PI_AE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

pi_ae_status fail(pi_ae_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

}  // namespace

void pi_ae::set_last_error(const std::string& msg) { g_last_error = msg; }

namespace {

struct HipError {
  hipError_t e;
  std::string what;
};

#define HIP_OR_THROW(call)                                                      \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) throw HipError{e_, std::string(#call) + ": " + hipGetErrorString(e_)}; \
  } while (0)

inline double bf(uint16_t v) {
  uint32_t u = uint32_t(v) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}
// fp64 -> bf16 bits, round to nearest even (through fp32, also RNE)
inline uint16_t bf16_of(double x) {
  const float f = float(x);
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return uint16_t(u >> 16);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Device allocations of one library object.  Each allocation carries a
// 256-byte guard on both sides filled with a fixed byte pattern, which
// check() reads back: a kernel that wrote past either end of a buffer leaves
// a changed guard.  PI_AE_FAIL_ALLOC=N (environment, read when the object is
// prepared) makes its N-th allocation fail as out of memory, so that tests
// can check that every failure path frees what was allocated before it.
constexpr size_t kGuardBytes = 256;
constexpr unsigned char kGuardByte = 0xA5;
// device bytes held by every live arena of the process (guards included)
std::atomic<int64_t> g_live_device_bytes{0};

struct DeviceArena {
  struct Block {
    char* base;      // the hipMalloc'ed range: guard, buffer, guard
    size_t bytes;    // buffer bytes (between the guards)
  };
  std::vector<Block> blocks;
  int count = 0, fail_at = 0;

  void arm_fault_injection() {
    count = 0;
    const char* e = std::getenv("PI_AE_FAIL_ALLOC");
    fail_at = e ? std::atoi(e) : 0;
  }
  template <class T>
  T* alloc(size_t n) {
    if (n == 0) n = 1;
    const size_t bytes = n * sizeof(T);
    if (++count == fail_at)
      throw HipError{hipErrorOutOfMemory, "injected failure of device allocation " + std::to_string(count) +
                                              " (PI_AE_FAIL_ALLOC)"};
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes + 2 * kGuardBytes);
    if (e != hipSuccess) throw HipError{e, "hipMalloc of " + std::to_string(bytes) + " bytes"};
    char* base = static_cast<char*>(p);
    blocks.push_back(Block{base, bytes});
    g_live_device_bytes += int64_t(bytes + 2 * kGuardBytes);
    e = hipMemset(base, kGuardByte, kGuardBytes);
    if (e == hipSuccess) e = hipMemset(base + kGuardBytes + bytes, kGuardByte, kGuardBytes);
    if (e != hipSuccess) throw HipError{e, "guard fill"};
    return reinterpret_cast<T*>(base + kGuardBytes);
  }
  // index of the first block whose guards changed, -1 if none; corrupt >= 0
  // first overwrites one byte right after that block's buffer (a host-side
  // write of the guard, to show that the check sees it)
  int check(int corrupt, hipError_t* err) {
    *err = hipSuccess;
    if (corrupt >= 0 && corrupt < int(blocks.size())) {
      *err = hipMemset(blocks[corrupt].base + kGuardBytes + blocks[corrupt].bytes, 0, 1);
      if (*err != hipSuccess) return -1;
    }
    std::vector<unsigned char> g(kGuardBytes);
    for (size_t i = 0; i < blocks.size(); ++i) {
      for (int side = 0; side < 2; ++side) {
        const char* src = side ? blocks[i].base + kGuardBytes + blocks[i].bytes : blocks[i].base;
        *err = hipMemcpy(g.data(), src, kGuardBytes, hipMemcpyDeviceToHost);
        if (*err != hipSuccess) return -1;
        for (unsigned char c : g)
          if (c != kGuardByte) return int(i);
      }
    }
    return -1;
  }
  void release() {
    for (const Block& b : blocks) {
      (void)hipFree(b.base);
      g_live_device_bytes -= int64_t(b.bytes + 2 * kGuardBytes);
    }
    blocks.clear();
  }
};

// Executable graphs of one library object, keyed by call shape.  At most
// kGraphCacheMax are kept (the least recently used is dropped), and each holds
// an event recorded after its latest launch, so that dropping it, and
// destroying the object, wait for that object's own work only.
constexpr size_t kGraphCacheMax = 8;

template <class Key>
struct GraphCache {
  struct Entry {
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;
    uint64_t used = 0;
  };
  std::map<Key, Entry> m;
  uint64_t tick = 0;

  Entry* find(const Key& k) {
    auto it = m.find(k);
    if (it == m.end()) return nullptr;
    it->second.used = ++tick;
    return &it->second;
  }
  // takes ownership of exec (destroyed here on failure)
  hipError_t insert(const Key& k, hipGraphExec_t exec, Entry** out) {
    if (m.size() >= kGraphCacheMax) {
      auto lru = m.begin();
      for (auto it = m.begin(); it != m.end(); ++it)
        if (it->second.used < lru->second.used) lru = it;
      drop(lru->second);
      m.erase(lru);
    }
    hipEvent_t ev = nullptr;
    const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipGraphExecDestroy(exec);
      return e;
    }
    Entry& en = m[k];
    en.exec = exec;
    en.done = ev;
    en.used = ++tick;
    *out = &en;
    return hipSuccess;
  }
  static hipError_t launch(Entry* en, hipStream_t s) { return hipGraphLaunch(en->exec, s); }
  // after the call's last work on s (the graph and anything enqueued after it)
  static hipError_t mark(Entry* en, hipStream_t s) { return hipEventRecord(en->done, s); }
  static void drop(Entry& en) {
    (void)hipEventSynchronize(en.done);  // a launch of it may still be in flight
    (void)hipGraphExecDestroy(en.exec);
    (void)hipEventDestroy(en.done);
  }
  void clear() {
    for (auto& kv : m) drop(kv.second);
    m.clear();
  }
};

// Captures what `enq` enqueues on `cap` into a new executable graph.
template <class F>
hipError_t capture_graph(hipStream_t cap, F&& enq, hipGraphExec_t* out) {
  hipGraph_t graph = nullptr;
  *out = nullptr;
  hipError_t e = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    const hipError_t e2 = enq();
    e = hipStreamEndCapture(cap, &graph);
    if (e2 != hipSuccess) e = e2;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(out, graph, nullptr, nullptr, 0);
  if (graph) (void)hipGraphDestroy(graph);
  return e;
}

}  // namespace

// The device memory one call of the loop works in: the residual stream and
// the GEMM operands, the call's packed K/V and key bias, its RoPE rows, valid
// prefix counts and argument block.  A context owns one (allocated when it is
// prepared); the allocation-free entry point carves one out of a fixed device
// array instead.
struct Workspace {
  float* h = nullptr;                       // [Mpad][1024] fp32 residual stream
  uint16_t *q = nullptr, *o = nullptr, *m = nullptr, *u = nullptr;
  uint16_t* o2 = nullptr;                   // second key range's partial attention output, then row statistics
  float* ssq = nullptr;                     // [Mpad][64] partial sums of h^2
  uint16_t *kp = nullptr, *vp = nullptr;    // packed K/V of every layer, one call
  float* kbias = nullptr;
  float2* rope_cs = nullptr;
  int* n_valid = nullptr;
  DevArgs* da = nullptr;
};

struct pi_ae_ctx {
  pi_ae_config cfg{};
  int device = 0;
  bool broken = false;
  DeviceArena arena;
  // prepared weights (device)
  uint16_t *w_qkv = nullptr, *w_o = nullptr, *w_gu = nullptr, *w_d = nullptr, *w_in = nullptr, *w_out = nullptr;
  float* b_in = nullptr;
  // pi0 variant: the encoder's output layer (swizzled), its bias, the encoder's
  // per-step input bias [S][1024] and a gate of ones
  uint16_t* w_to = nullptr;
  float *b_to = nullptr, *enc_bias = nullptr, *ones = nullptr;
  // tables (device), kernel column order
  float *attn_s1 = nullptr, *attn_g = nullptr, *c_qkv = nullptr, *ffn_s1 = nullptr, *ffn_g = nullptr,
        *c_gu = nullptr, *fin_s1 = nullptr, *c_out = nullptr;
  double* inv_freq = nullptr;
  Workspace ws;
  int nkb_max = 0;
  int Mmax = 0, Mpad = 0;
  // host copies of the tables in natural column order (debug export)
  std::vector<float> tab[10];
  hipStream_t cap = nullptr;
  GraphCache<std::pair<int, int>> graphs;

  template <class T>
  T* dalloc(size_t n) {
    return arena.alloc<T>(n);
  }
  void release() {
    graphs.clear();
    arena.release();
    if (cap) (void)hipStreamDestroy(cap);
    cap = nullptr;
  }
};

namespace {

// ------------------------------------------------------------------ validation
pi_ae_status check_config(const pi_ae_config* c) {
  if (c->width != kD || c->mlp_dim != kF || c->num_heads != kH || c->num_kv_heads != 1 || c->head_dim != kHd ||
      c->action_dim != kA)
    return fail(PI_AE_EUNSUPPORTED,
                "kernels implement width 1024, mlp_dim 4096, 8 heads, 1 KV head, head_dim 256, action_dim 32");
  if (c->num_layers < 1 || c->num_layers > 64) return fail(PI_AE_EINVAL, "num_layers must be in [1, 64]");
  if (c->num_steps < 1 || c->num_steps > 64) return fail(PI_AE_EINVAL, "num_steps must be in [1, 64]");
  if (c->chunk_len < 1 || c->chunk_len > 256) return fail(PI_AE_EINVAL, "chunk_len must be in [1, 256]");
  if (c->max_batch < 1 || c->max_batch > 1024) return fail(PI_AE_EINVAL, "max_batch must be in [1, 1024]");
  if (c->max_batch * c->chunk_len > 65536)
    return fail(PI_AE_EINVAL, "max_batch * chunk_len (rows per GEMM) must be at most 65536");
  if (c->max_prefix_len < 0 || c->max_prefix_len > 8192)
    return fail(PI_AE_EINVAL, "max_prefix_len must be in [0, 8192]");
  if (!std::isfinite(c->t0) || !std::isfinite(c->dt)) return fail(PI_AE_EINVAL, "t0 and dt must be finite");
  if (!(c->rope_base > 0.f) || !std::isfinite(c->rope_base)) return fail(PI_AE_EINVAL, "rope_base must be > 0");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps)) return fail(PI_AE_EINVAL, "rms_eps must be >= 0");
  if (c->final_norm != 0 && c->final_norm != 1) return fail(PI_AE_EINVAL, "final_norm must be 0 or 1");
  if (c->variant != 0 && c->variant != 1) return fail(PI_AE_EINVAL, "variant must be 0 (pi0.5) or 1 (pi0)");
  return PI_AE_OK;
}

pi_ae_status check_weights(const pi_ae_config* c, const pi_ae_weights* w) {
  auto need = [](const pi_ae_linear& l, bool bias, const char* name) -> pi_ae_status {
    if (!l.w) return fail(PI_AE_EINVAL, std::string("weight ") + name + ".w is NULL");
    if (bias && !l.b) return fail(PI_AE_EINVAL, std::string("weight ") + name + ".b is NULL");
    return PI_AE_OK;
  };
  pi_ae_status s;
  if (c->variant == 1) {
    if ((s = need(w->action_in, true, "action_in")) || (s = need(w->action_time_in, true, "action_time_in")) ||
        (s = need(w->action_time_out, true, "action_time_out")) || (s = need(w->action_out, true, "action_out")))
      return s;
    if (c->final_norm && !w->final_norm) return fail(PI_AE_EINVAL, "final_norm (gamma) is NULL");
    if (!w->layers) return fail(PI_AE_EINVAL, "layers is NULL");
    for (int l = 0; l < c->num_layers; ++l) {
      const pi_ae_layer_weights& L = w->layers[l];
      if (!L.attn_norm || !L.ffn_norm)
        return fail(PI_AE_EINVAL, "attn_norm / ffn_norm is NULL (layer " + std::to_string(l) + ")");
      if ((s = need(L.q, false, "q")) || (s = need(L.k, false, "k")) || (s = need(L.v, false, "v")) ||
          (s = need(L.o, false, "o")) || (s = need(L.gate, false, "gate")) || (s = need(L.up, false, "up")) ||
          (s = need(L.down, false, "down")))
        return fail(s, g_last_error + " (layer " + std::to_string(l) + ")");
    }
    return PI_AE_OK;
  }
  if ((s = need(w->action_in, true, "action_in")) || (s = need(w->time_in, true, "time_in")) ||
      (s = need(w->time_out, true, "time_out")) || (s = need(w->action_out, true, "action_out")))
    return s;
  if (c->final_norm && (s = need(w->final_mod, true, "final_mod"))) return s;
  if (!w->layers) return fail(PI_AE_EINVAL, "layers is NULL");
  for (int l = 0; l < c->num_layers; ++l) {
    const pi_ae_layer_weights& L = w->layers[l];
    if ((s = need(L.attn_mod, true, "attn_mod")) || (s = need(L.q, false, "q")) || (s = need(L.k, false, "k")) ||
        (s = need(L.v, false, "v")) || (s = need(L.o, false, "o")) || (s = need(L.ffn_mod, true, "ffn_mod")) ||
        (s = need(L.gate, false, "gate")) || (s = need(L.up, false, "up")) || (s = need(L.down, false, "down")))
      return fail(s, g_last_error + " (layer " + std::to_string(l) + ")");
  }
  return PI_AE_OK;
}

// ------------------------------------------------------------------ host math (fp64)
// Sinusoidal timestep embedding: dim/2 sines then dim/2 cosines, periods
// geometric from 4e-3 to 4.0 (the pages name the embedding but not its
// frequencies; this is the reading the library documents and tests).
std::vector<double> time_embedding(double t, int dim) {
  const int half = dim / 2;
  std::vector<double> e(dim);
  for (int i = 0; i < half; ++i) {
    const double frac = double(i) / double(half - 1);
    const double period = 4e-3 * std::pow(4.0 / 4e-3, frac);
    const double ang = 2.0 * M_PI * t / period;
    e[i] = std::sin(ang);
    e[half + i] = std::cos(ang);
  }
  return e;
}

inline double silu(double x) { return x / (1.0 + std::exp(-x)); }

// y = W x + b for a bf16 W [n][k]
std::vector<double> matvec(const uint16_t* W, const uint16_t* b, const std::vector<double>& x, int n, int k) {
  std::vector<double> y(n);
  for (int i = 0; i < n; ++i) {
    const uint16_t* row = W + size_t(i) * k;
    double acc = b ? bf(b[i]) : 0.0;
    for (int j = 0; j < k; ++j) acc += bf(row[j]) * x[j];
    y[i] = acc;
  }
  return y;
}

// Swizzle rows `perm` of W[N][K] into MFMA B-operand fragments (see frag_offset).
void swizzle(const uint16_t* W, int K, const std::vector<int>& perm, uint16_t* out) {
  const int NBk = int(perm.size()) / 16, KB = K / 32;
  for (int nb = 0; nb < NBk; ++nb)
    for (int kb = 0; kb < KB; ++kb) {
      uint16_t* frag = out + frag_offset(nb, kb, KB);
      for (int lane = 0; lane < 64; ++lane) {
        const uint16_t* src = W + size_t(perm[nb * 16 + lane % 16]) * K + kb * 32 + 8 * (lane / 16);
        std::memcpy(frag + lane * 8, src, 16);
      }
    }
}

// Column order of the fused QKV GEMM: workgroup j owns n-blocks 2j, 2j+1.
// Q head h (j = 8h + pb) and K_s (j = 64 + pb): the two blocks are head-dim
// channels pb*16 + [0,16) and 128 + pb*16 + [0,16), so each output tile holds
// whole RoPE pairs (i, i+128).  V_s (j = 72..79): 32 consecutive channels.
// Natural fused index: q rows 0..2047, k rows 2048..2303, v rows 2304..2559.
std::vector<int> qkv_perm() {
  std::vector<int> p(kNqkv);
  for (int j = 0; j < kNqkv / 32; ++j)
    for (int nbi = 0; nbi < 2; ++nbi)
      for (int c = 0; c < 16; ++c) {
        int nat;
        if (j < 64) nat = (j >> 3) * kHd + nbi * kRopeHalf + (j & 7) * 16 + c;
        else if (j < 72) nat = kH * kHd + nbi * kRopeHalf + (j - 64) * 16 + c;
        else nat = kH * kHd + kHd + (j - 72) * 32 + nbi * 16 + c;
        p[(2 * j + nbi) * 16 + c] = nat;
      }
  return p;
}

// Fused gate|up: workgroup j owns gate rows 16j.. (n-block 2j) and the same
// up rows (n-block 2j+1).  Natural fused index: gate f -> f, up f -> F + f.
std::vector<int> gu_perm(int F = kF) {
  std::vector<int> p(2 * F);
  for (int j = 0; j < F / 16; ++j)
    for (int c = 0; c < 16; ++c) {
      p[(2 * j) * 16 + c] = 16 * j + c;
      p[(2 * j + 1) * 16 + c] = F + 16 * j + c;
    }
  return p;
}

template <class F>
void parallel_for(int n, F&& fn) {
  int nt = std::max(1, std::min<int>(n, int(std::thread::hardware_concurrency())));
  nt = std::min(nt, 16);
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int i = t; i < n; i += nt) fn(i);
    });
  for (auto& x : th) x.join();
}

// The fp64 host half of the preparation: tables in natural column order
// (0 attn 1+scale, 1 attn gate, 2 ffn 1+scale, 3 ffn gate, 4 final 1+scale,
// 5 c_out, 6 c_qkv, 7 c_gu, 8 timesteps, 9 cond).
// pi0 ("Running VLAs at Real-time Speed" notes, section How; blog section
// 3.2): the norm scales gamma as the (1 + scale) tables (gates 1, shifts 0, so
// c_qkv = c_gu = 0 and c_out = b_out), and the action-time encoder's
// per-step bias before its SiLU, W_ti[:, :D] b_in + W_ti[:, D:] emb(t_k) + b_ti.
void compute_tables_pi0(const pi_ae_config& cfg, const pi_ae_weights* w, const std::vector<double>& ts,
                        std::vector<float>* tab) {
  const int L = cfg.num_layers, S = cfg.num_steps;
  tab[0].assign(size_t(S) * L * kD, 0.f); tab[1].assign(size_t(S) * L * kD, 1.f);
  tab[2].assign(size_t(S) * L * kD, 0.f); tab[3].assign(size_t(S) * L * kD, 1.f);
  for (int k = 0; k < S; ++k)
    for (int l = 0; l < L; ++l)
      for (int i = 0; i < kD; ++i) {
        tab[0][(size_t(k) * L + l) * kD + i] = float(bf(w->layers[l].attn_norm[i]));
        tab[2][(size_t(k) * L + l) * kD + i] = float(bf(w->layers[l].ffn_norm[i]));
      }
  tab[4].assign(size_t(S) * kD, 1.f);
  if (cfg.final_norm)
    for (int k = 0; k < S; ++k)
      for (int i = 0; i < kD; ++i) tab[4][size_t(k) * kD + i] = float(bf(w->final_norm[i]));
  tab[5].resize(size_t(S) * kA);
  for (int k = 0; k < S; ++k)
    for (int a = 0; a < kA; ++a) tab[5][size_t(k) * kA + a] = float(bf(w->action_out.b[a]));
  tab[6].assign(size_t(S) * L * kNqkv, 0.f);
  tab[7].assign(size_t(S) * L * kNgu, 0.f);
  tab[8].assign(ts.begin(), ts.end());
  tab[9].resize(size_t(S) * kD);
  std::vector<double> bin(kD);
  for (int j = 0; j < kD; ++j) bin[j] = bf(w->action_in.b[j]);
  parallel_for(S, [&](int k) {
    const std::vector<double> emb = time_embedding(ts[k], kD);
    for (int i = 0; i < kD; ++i) {
      const uint16_t* row = w->action_time_in.w + size_t(i) * 2 * kD;
      double acc = bf(w->action_time_in.b[i]);
      for (int j = 0; j < kD; ++j) acc += bf(row[j]) * bin[j] + bf(row[kD + j]) * emb[j];
      tab[9][size_t(k) * kD + i] = float(acc);
    }
  });
}

void compute_tables(const pi_ae_config& cfg, const pi_ae_weights* w, std::vector<float>* tab) {
  const int L = cfg.num_layers, S = cfg.num_steps;
  // timesteps t_k = fp32(t0 + k dt), evaluated in fp64
  std::vector<double> ts(S);
  for (int k = 0; k < S; ++k) ts[k] = double(float(double(cfg.t0) + k * double(cfg.dt)));
  if (cfg.variant == 1) return compute_tables_pi0(cfg, w, ts, tab);
  // time MLP: cond_k = SiLU(W_out SiLU(W_in emb + b_in) + b_out)
  std::vector<std::vector<double>> cond(S);
  parallel_for(S, [&](int k) {
    std::vector<double> a = matvec(w->time_in.w, w->time_in.b, time_embedding(ts[k], kD), kD, kD);
    for (double& v : a) v = silu(v);
    std::vector<double> c = matvec(w->time_out.w, w->time_out.b, a, kD, kD);
    for (double& v : c) v = silu(v);
    cond[k] = std::move(c);
  });
  // per (step, layer) modulation and shift-fold biases, natural order
  auto& t_as1 = tab[0]; auto& t_ag = tab[1]; auto& t_fs1 = tab[2]; auto& t_fg = tab[3];
  auto& t_fin = tab[4]; auto& t_cout = tab[5]; auto& t_cqkv = tab[6]; auto& t_cgu = tab[7];
  t_as1.assign(size_t(S) * L * kD, 0.f); t_ag = t_as1; t_fs1 = t_as1; t_fg = t_as1;
  t_cqkv.assign(size_t(S) * L * kNqkv, 0.f);
  t_cgu.assign(size_t(S) * L * kNgu, 0.f);
  parallel_for(L, [&](int l) {
    const pi_ae_layer_weights& Lw = w->layers[l];
    std::vector<std::vector<double>> sh_a(S), sh_f(S);
    for (int k = 0; k < S; ++k) {
      std::vector<double> ma = matvec(Lw.attn_mod.w, Lw.attn_mod.b, cond[k], 3 * kD, kD);
      std::vector<double> mf = matvec(Lw.ffn_mod.w, Lw.ffn_mod.b, cond[k], 3 * kD, kD);
      const size_t o = (size_t(k) * L + l) * kD;
      for (int i = 0; i < kD; ++i) {
        t_as1[o + i] = float(1.0 + ma[i]);
        t_ag[o + i] = float(ma[2 * kD + i]);
        t_fs1[o + i] = float(1.0 + mf[i]);
        t_fg[o + i] = float(mf[2 * kD + i]);
      }
      sh_a[k].assign(ma.begin() + kD, ma.begin() + 2 * kD);
      sh_f[k].assign(mf.begin() + kD, mf.begin() + 2 * kD);
    }
    // c = shift @ W^T for every fused output column, all steps per weight row
    std::vector<double> row(kD);
    auto fold = [&](const uint16_t* W, int nrows, const std::vector<std::vector<double>>& sh, std::vector<float>& dst,
                    int width, int col0) {
      for (int n = 0; n < nrows; ++n) {
        for (int j = 0; j < kD; ++j) row[j] = bf(W[size_t(n) * kD + j]);
        for (int k = 0; k < S; ++k) {
          double acc = 0.0;
          for (int j = 0; j < kD; ++j) acc += row[j] * sh[k][j];
          dst[(size_t(k) * L + l) * width + col0 + n] = float(acc);
        }
      }
    };
    fold(Lw.q.w, kH * kHd, sh_a, t_cqkv, kNqkv, 0);
    fold(Lw.k.w, kHd, sh_a, t_cqkv, kNqkv, kH * kHd);
    fold(Lw.v.w, kHd, sh_a, t_cqkv, kNqkv, kH * kHd + kHd);
    fold(Lw.gate.w, kF, sh_f, t_cgu, kNgu, 0);
    fold(Lw.up.w, kF, sh_f, t_cgu, kNgu, kF);
  });
  // final norm table and c_out = shift_f @ W_out^T + b_out
  t_fin.assign(size_t(S) * kD, 1.f);
  t_cout.assign(size_t(S) * kA, 0.f);
  for (int k = 0; k < S; ++k) {
    std::vector<double> shf(kD, 0.0);
    if (cfg.final_norm) {
      std::vector<double> mfin = matvec(w->final_mod.w, w->final_mod.b, cond[k], 3 * kD, kD);
      for (int i = 0; i < kD; ++i) t_fin[size_t(k) * kD + i] = float(1.0 + mfin[i]);
      shf.assign(mfin.begin() + kD, mfin.begin() + 2 * kD);
    }
    std::vector<double> c = matvec(w->action_out.w, w->action_out.b, shf, kA, kD);
    for (int a = 0; a < kA; ++a) t_cout[size_t(k) * kA + a] = float(c[a]);
  }
  tab[8].assign(ts.begin(), ts.end());
  tab[9].resize(size_t(S) * kD);
  for (int k = 0; k < S; ++k)
    for (int i = 0; i < kD; ++i) tab[9][size_t(k) * kD + i] = float(cond[k][i]);
}

void prepare(pi_ae_ctx* ctx, const pi_ae_weights* w) {
  const pi_ae_config& cfg = ctx->cfg;
  const int L = cfg.num_layers, T = cfg.chunk_len;
  compute_tables(cfg, w, ctx->tab);
  auto& t_as1 = ctx->tab[0]; auto& t_ag = ctx->tab[1]; auto& t_fs1 = ctx->tab[2]; auto& t_fg = ctx->tab[3];
  auto& t_fin = ctx->tab[4]; auto& t_cout = ctx->tab[5]; auto& t_cqkv = ctx->tab[6]; auto& t_cgu = ctx->tab[7];

  // ---- device weights
  const std::vector<int> pq = qkv_perm(), pg = gu_perm();
  std::vector<int> pid(kD);
  for (int i = 0; i < kD; ++i) pid[i] = i;
  const size_t n_qkv = size_t(kNqkv) * kD, n_o = size_t(kD) * kH * kHd, n_gu = size_t(kNgu) * kD,
               n_d = size_t(kD) * kF;
  ctx->w_qkv = ctx->dalloc<uint16_t>(n_qkv * L);
  ctx->w_o = ctx->dalloc<uint16_t>(n_o * L);
  ctx->w_gu = ctx->dalloc<uint16_t>(n_gu * L);
  ctx->w_d = ctx->dalloc<uint16_t>(n_d * L);
  {
    std::vector<uint16_t> fused(std::max(n_qkv, n_gu)), sw(std::max(std::max(n_qkv, n_gu), std::max(n_o, n_d)));
    for (int l = 0; l < L; ++l) {
      const pi_ae_layer_weights& Lw = w->layers[l];
      std::memcpy(fused.data(), Lw.q.w, sizeof(uint16_t) * kH * kHd * kD);
      std::memcpy(fused.data() + size_t(kH) * kHd * kD, Lw.k.w, sizeof(uint16_t) * kHd * kD);
      std::memcpy(fused.data() + size_t(kH + 1) * kHd * kD, Lw.v.w, sizeof(uint16_t) * kHd * kD);
      swizzle(fused.data(), kD, pq, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_qkv + n_qkv * l, sw.data(), n_qkv * 2, hipMemcpyHostToDevice));
      swizzle(Lw.o.w, kH * kHd, pid, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_o + n_o * l, sw.data(), n_o * 2, hipMemcpyHostToDevice));
      std::memcpy(fused.data(), Lw.gate.w, sizeof(uint16_t) * kF * kD);
      std::memcpy(fused.data() + size_t(kF) * kD, Lw.up.w, sizeof(uint16_t) * kF * kD);
      swizzle(fused.data(), kD, pg, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_gu + n_gu * l, sw.data(), n_gu * 2, hipMemcpyHostToDevice));
      swizzle(Lw.down.w, kF, pid, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_d + n_d * l, sw.data(), n_d * 2, hipMemcpyHostToDevice));
    }
  }
  ctx->w_in = ctx->dalloc<uint16_t>(size_t(kD) * kA);
  if (cfg.variant == 1) {
    // the encoder's input layer folded with action_in_proj: W_ti[:, :D] W_in
    // (fp64, rounded to bf16 once); its output layer swizzled like W_o
    std::vector<uint16_t> wf(size_t(kD) * kA);
    parallel_for(kD, [&](int i) {
      const uint16_t* row = w->action_time_in.w + size_t(i) * 2 * kD;
      for (int a = 0; a < kA; ++a) {
        double acc = 0.0;
        for (int j = 0; j < kD; ++j) acc += bf(row[j]) * bf(w->action_in.w[size_t(j) * kA + a]);
        wf[size_t(i) * kA + a] = bf16_of(acc);
      }
    });
    HIP_OR_THROW(hipMemcpy(ctx->w_in, wf.data(), wf.size() * 2, hipMemcpyHostToDevice));
    std::vector<uint16_t> sw(size_t(kD) * kD);
    swizzle(w->action_time_out.w, kD, pid, sw.data());
    ctx->w_to = ctx->dalloc<uint16_t>(sw.size());
    HIP_OR_THROW(hipMemcpy(ctx->w_to, sw.data(), sw.size() * 2, hipMemcpyHostToDevice));
    std::vector<float> bto(kD), ones(kD, 1.f);
    for (int i = 0; i < kD; ++i) bto[i] = float(bf(w->action_time_out.b[i]));
    ctx->b_to = ctx->dalloc<float>(kD);
    HIP_OR_THROW(hipMemcpy(ctx->b_to, bto.data(), kD * 4, hipMemcpyHostToDevice));
    ctx->ones = ctx->dalloc<float>(kD);
    HIP_OR_THROW(hipMemcpy(ctx->ones, ones.data(), kD * 4, hipMemcpyHostToDevice));
  } else {
    HIP_OR_THROW(hipMemcpy(ctx->w_in, w->action_in.w, size_t(kD) * kA * 2, hipMemcpyHostToDevice));
  }
  ctx->w_out = ctx->dalloc<uint16_t>(size_t(kA) * kD);
  HIP_OR_THROW(hipMemcpy(ctx->w_out, w->action_out.w, size_t(kA) * kD * 2, hipMemcpyHostToDevice));
  {
    std::vector<float> bin(kD);
    for (int i = 0; i < kD; ++i) bin[i] = float(bf(w->action_in.b[i]));
    ctx->b_in = ctx->dalloc<float>(kD);
    HIP_OR_THROW(hipMemcpy(ctx->b_in, bin.data(), kD * 4, hipMemcpyHostToDevice));
  }
  // ---- device tables in kernel column order
  auto upload = [&](const std::vector<float>& v) {
    float* d = ctx->dalloc<float>(v.size());
    HIP_OR_THROW(hipMemcpy(d, v.data(), v.size() * 4, hipMemcpyHostToDevice));
    return d;
  };
  auto permute = [&](const std::vector<float>& nat, int width, const std::vector<int>& perm) {
    std::vector<float> out(nat.size());
    for (size_t r = 0; r < nat.size() / width; ++r)
      for (int i = 0; i < width; ++i) out[r * width + i] = nat[r * width + perm[i]];
    return out;
  };
  ctx->attn_s1 = upload(t_as1);
  ctx->attn_g = upload(t_ag);
  ctx->ffn_s1 = upload(t_fs1);
  ctx->ffn_g = upload(t_fg);
  ctx->fin_s1 = upload(t_fin);
  ctx->c_out = upload(t_cout);
  ctx->c_qkv = upload(permute(t_cqkv, kNqkv, pq));
  ctx->c_gu = upload(permute(t_cgu, kNgu, pg));
  if (cfg.variant == 1) ctx->enc_bias = upload(ctx->tab[9]);
  // RoPE inverse frequencies base^(-2i/256) in fp64; the pack kernel turns
  // them into the cos/sin rows of the call's suffix positions
  {
    std::vector<double> inv(kRopeHalf);
    for (int i = 0; i < kRopeHalf; ++i) inv[i] = std::pow(double(cfg.rope_base), -2.0 * i / kHd);
    ctx->inv_freq = ctx->dalloc<double>(kRopeHalf);
    HIP_OR_THROW(hipMemcpy(ctx->inv_freq, inv.data(), kRopeHalf * 8, hipMemcpyHostToDevice));
  }
  // ---- workspaces (zeroed once; padded rows are never written)
  ctx->Mmax = cfg.max_batch * T;
  ctx->Mpad = (ctx->Mmax + 255) / 256 * 256;  // whole 256-row tiles of the wide gate/up GEMM
  const size_t Mp = size_t(ctx->Mpad);
  ctx->ws.h = ctx->dalloc<float>(Mp * kD);
  ctx->ws.q = ctx->dalloc<uint16_t>(Mp * kH * kHd);
  ctx->nkb_max = (cfg.max_prefix_len + T + 31) / 32;
  const size_t npack = size_t(L) * cfg.max_batch * ctx->nkb_max * 8192;
  ctx->ws.kp = ctx->dalloc<uint16_t>(npack);
  ctx->ws.vp = ctx->dalloc<uint16_t>(npack);
  ctx->ws.kbias = ctx->dalloc<float>(size_t(cfg.max_batch) * ctx->nkb_max * 32);
  ctx->ws.o = ctx->dalloc<uint16_t>(Mp * kH * kHd);
  ctx->ws.rope_cs = ctx->dalloc<float2>(Mp * kRopeHalf);
  ctx->ws.u = ctx->dalloc<uint16_t>(Mp * kD);
  ctx->ws.ssq = ctx->dalloc<float>(Mp * (kD / 16));
  ctx->ws.m = ctx->dalloc<uint16_t>(Mp * kF);
  ctx->ws.n_valid = ctx->dalloc<int>(cfg.max_batch);
  ctx->ws.da = ctx->dalloc<DevArgs>(1);
  ctx->ws.o2 = ctx->dalloc<uint16_t>(Mp * kH * kHd + Mp * kH * 4 * 2);  // + row statistics (fp32)
  HIP_OR_THROW(hipMemset(ctx->ws.h, 0, Mp * kD * 4));
  HIP_OR_THROW(hipMemset(ctx->ws.q, 0, Mp * kH * kHd * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.kp, 0, npack * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.vp, 0, npack * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.o, 0, Mp * kH * kHd * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.o2, 0, (Mp * kH * kHd + Mp * kH * 4 * 2) * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.u, 0, Mp * kD * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.ssq, 0, Mp * (kD / 16) * 4));
  HIP_OR_THROW(hipMemset(ctx->ws.m, 0, Mp * kF * 2));
  HIP_OR_THROW(hipMemset(ctx->ws.n_valid, 0, cfg.max_batch * 4));
  HIP_OR_THROW(hipMemset(ctx->ws.da, 0, sizeof(DevArgs)));
  HIP_OR_THROW(hipStreamCreateWithFlags(&ctx->cap, hipStreamNonBlocking));
  HIP_OR_THROW(hipDeviceSynchronize());
}

// ------------------------------------------------------------------ step sequence
// Attention key split: at small M (the weight-streaming GEMM path) and long
// key sequences each query block's keys go to two workgroups and the O
// projection merges the halves.  Measured on the 10-step loop: -5.5% at 28
// key blocks, -1.9% at 18, +1.4% at 10 (the merge in the O projection costs
// more than the shorter key stream saves).
constexpr int kAttnSplitMinBlocks = 16;
static int attn_ksplit(int M, int nkb) { return M < kTiledMinRows && nkb >= kAttnSplitMinBlocks ? 2 : 1; }

// Phases: 0 = step input (k_io), 1 = QKV, 2 = attention, 3 = O, 4 = gate/up, 5 = down.
// stop(step, layer, phase) returns true after the named phase has been enqueued.
struct StopAt {
  int step = -1, layer = -1, phase = -1;
  bool hit(int k, int l, int ph) const { return k == step && (ph == 0 ? true : l == layer) && ph == phase; }
};

Prefetch slices(const void* base, size_t bytes, int count) { return Prefetch{base, uint32_t(bytes), count}; }
Prefetch broadcast(const void* base, size_t bytes) { return Prefetch{base, uint32_t(bytes), 0}; }

// L2 warm-up plan of the streaming (small-M) path: spare workgroups of a
// kernel read what a later kernel streams, into the L2 of the XCD whose
// workgroups will read it (see Prefetch).  Only kernels that leave CUs idle
// host warm-ups (a prefetching workgroup that shares a CU with a main one
// slows it more than the warm-up saves): the step input, QKV (80 or 160
// workgroups) and attention (32 per episode).  Only data that no kernel of
// the loop writes is prefetched: weights, and whole prefix blocks of K/V.
//   step input     -> layer 0 QKV weights
//   QKV(l)         -> layer l prefix K and V (batch 1)
//   attention(l)   -> layer l O and gate/up weights
PrefetchSet warm_plan(const pi_ae_ctx* ctx, const Workspace& ws, int B, int P, int k, int l, int phase) {
  const pi_ae_config& cfg = ctx->cfg;
  const int T = cfg.chunk_len;
  PrefetchSet pf{};
  if (B * T >= kTiledMinRows) return pf;
  const size_t qkv_slice = size_t(32) * kD * 2;
  switch (phase) {
    case 0:
      if (k < cfg.num_steps) {
        pf.r[0] = slices(ctx->w_qkv, qkv_slice, kNqkv / 32);
        pf.nwg = 80;
      }
      break;
    case 1: {
      const int nkb = (P + T + 31) / 32, full = P / 32;
      if (B == 1 && full > 0) {
        const size_t off = size_t(l) * nkb * 8192;
        pf.r[0] = broadcast(ws.kp + off, size_t(full) * 8192 * 2);
        pf.r[1] = broadcast(ws.vp + off, size_t(full) * 8192 * 2);
        pf.nwg = 32;
      }
      break;
    }
    case 2:
      pf.r[0] = slices(ctx->w_o + size_t(kD) * kH * kHd * l, size_t(16) * kH * kHd * 2, kD / 16);
      pf.r[1] = slices(ctx->w_gu + size_t(kNgu) * kD * l, size_t(32) * kD * 2, kNgu / 32);
      pf.nwg = 160;
      break;
  }
  return pf;
}

// Launch one phase of one (step, layer); phase 0 is the step-boundary kernel
// of step k (k == num_steps: the final output projection and Euler update).
hipError_t launch_phase(pi_ae_ctx* ctx, const Workspace& ws, int B, int P, hipStream_t s, int k, int l,
                        int phase,
                        const KernelTiming* t = nullptr) {
  const pi_ae_config& cfg = ctx->cfg;
  const int L = cfg.num_layers, S = cfg.num_steps, T = cfg.chunk_len, M = B * T;
  const size_t kl = size_t(k) * L + l;
  const PrefetchSet pf = warm_plan(ctx, ws, B, P, k, l, phase);
  switch (phase) {
    case 0: {
      IoParams io{};
      io.pf = pf;
      io.da = ws.da;
      io.h = ws.h;
      io.w_in = ctx->w_in;
      io.b_in = ctx->b_in;
      io.w_out = ctx->w_out;
      io.dt = cfg.dt;
      io.eps = cfg.rms_eps;
      io.M = M;
      io.do_out = k > 0;
      io.do_in = k < S;
      io.from_noise = k == 0;
      io.fin_s1 = (k > 0 && cfg.final_norm) ? ctx->fin_s1 + size_t(k - 1) * kD : nullptr;
      io.c_out = k > 0 ? ctx->c_out + size_t(k - 1) * kA : nullptr;
      io.s1_next = k < S ? ctx->attn_s1 + size_t(k) * L * kD : nullptr;
      io.u_out = ws.u;
      io.ssq_out = ws.ssq;
      if (cfg.variant == 1) {  // pi0: the action-time encoder, then its output layer
        io.enc = 1;
        io.h_init = ctx->b_to;
        io.u_out = ws.o;
        io.b_in = k < S ? ctx->enc_bias + size_t(k) * kD : ctx->b_to;
        hipError_t e = launch_io(io, s, t);
        if (e != hipSuccess || k >= S) return e;
        GemmParams g{};
        g.M = M;
        g.w = ctx->w_to;
        g.a_frag = ws.o;
        g.gate = ctx->ones;
        g.h_out = ws.h;
        g.s1_next = ctx->attn_s1 + size_t(k) * L * kD;
        g.u_out = ws.u;
        g.ssq_out = ws.ssq;
        return launch_enc(g, s);
      }
      return launch_io(io, s, t);
    }
    case 1:
    case 4: {
      GemmParams g{};
      g.pf = pf;
      g.M = M;
      g.eps = cfg.rms_eps;
      g.T = T;
      g.rope_cs = ws.rope_cs;
      g.a_frag = ws.u;
      g.ssq = ws.ssq;
      if (phase == 1) {
        const int nkb = (P + T + 31) / 32;
        g.w = ctx->w_qkv + size_t(kNqkv) * kD * l;
        g.bias = ctx->c_qkv + kl * kNqkv;
        g.q_out = ws.q;
        g.P = P;
        g.nkb = nkb;
        g.kp = ws.kp + size_t(l) * B * nkb * 8192;
        g.vp = ws.vp + size_t(l) * B * nkb * 8192;
        return launch_qkv(g, s, t);
      }
      g.w = ctx->w_gu + size_t(kNgu) * kD * l;
      g.bias = ctx->c_gu + kl * kNgu;
      g.m_out = ws.m;
      return launch_gu(g, s, t);
    }
    case 2: {
      AttnParams a{};
      a.pf = pf;
      const int nkb = (P + T + 31) / 32;
      a.q = ws.q;
      a.kp = ws.kp + size_t(l) * B * nkb * 8192;
      a.vp = ws.vp + size_t(l) * B * nkb * 8192;
      a.kbias = ws.kbias;
      a.o = ws.o;
      a.o2 = attn_ksplit(M, nkb) == 2 ? ws.o2 : nullptr;
      a.B = B;
      a.T = T;
      a.P = P;
      a.nkb = nkb;
      return launch_attn(a, s, t);
    }
    case 3:
    case 5: {
      GemmParams g{};
      g.pf = pf;
      g.M = M;
      g.h_out = ws.h;
      g.u_out = ws.u;
      g.ssq_out = ws.ssq;
      if (phase == 3) {  // next: this layer's gate/up
        g.w = ctx->w_o + size_t(kD) * kH * kHd * l;
        g.a_frag = ws.o;
        if (attn_ksplit(M, (P + T + 31) / 32) == 2) {
          g.a_frag2 = ws.o2;
          g.astat = attn_row_stats(ws.o2, M);
        }
        g.gate = ctx->attn_g + kl * kD;
        g.s1_next = ctx->ffn_s1 + kl * kD;
        return launch_o(g, s, t);
      }
      // next: the following layer's QKV, or (last layer) the step boundary
      g.w = ctx->w_d + size_t(kD) * kF * l;
      g.a_frag = ws.m;
      g.gate = ctx->ffn_g + kl * kD;
      g.s1_next = (l + 1 < L) ? ctx->attn_s1 + (kl + 1) * kD : nullptr;
      return launch_down(g, s, t);
    }
  }
  return hipErrorInvalidValue;
}

// timed_phase / timing: launch i of that phase (in loop order) gets timing[i].
hipError_t enqueue(pi_ae_ctx* ctx, const Workspace& ws, int B, int P, hipStream_t s, const StopAt& stop,
                   int timed_phase = -1, const KernelTiming* timing = nullptr) {
  const int L = ctx->cfg.num_layers, S = ctx->cfg.num_steps;
  hipError_t e;
  PackParams pp{};
  pp.da = ws.da;
  pp.n_valid = ws.n_valid;
  pp.inv_freq = ctx->inv_freq;
  pp.rope_cs = ws.rope_cs;
  pp.kp = ws.kp;
  pp.vp = ws.vp;
  pp.kbias = ws.kbias;
  pp.B = B;
  pp.P = P;
  pp.T = ctx->cfg.chunk_len;
  pp.nkb = (P + pp.T + 31) / 32;
  if ((e = launch_pack(pp, L, s)) != hipSuccess) return e;
  int n_timed = 0;
  auto tm = [&](int ph) { return (timing && ph == timed_phase) ? &timing[n_timed++] : nullptr; };
  for (int k = 0; k <= S; ++k) {
    if ((e = launch_phase(ctx, ws, B, P, s, k, 0, 0, tm(0))) != hipSuccess) return e;
    if (stop.hit(k, 0, 0) || k == S) return hipSuccess;
    for (int l = 0; l < L; ++l)
      for (int ph = 1; ph <= 5; ++ph) {
        if ((e = launch_phase(ctx, ws, B, P, s, k, l, ph, tm(ph))) != hipSuccess) return e;
        if (stop.hit(k, l, ph)) return hipSuccess;
      }
  }
  return hipSuccess;
}

pi_ae_status check_call(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise, const float* actions,
                        int32_t batch) {
  if (!ctx) return fail(PI_AE_EINVAL, "ctx is NULL");
  if (ctx->broken) return fail(PI_AE_ESTATE, "context is unusable after an earlier failure");
  if (!kv) return fail(PI_AE_EINVAL, "kv is NULL");
  if (batch < 0 || batch > ctx->cfg.max_batch)
    return fail(PI_AE_EINVAL, "batch " + std::to_string(batch) + " outside [0, max_batch]");
  if (kv->prefix_len < 0 || kv->prefix_len > ctx->cfg.max_prefix_len)
    return fail(PI_AE_EINVAL, "prefix_len " + std::to_string(kv->prefix_len) + " outside [0, max_prefix_len]");
  if (batch == 0) return PI_AE_OK;
  if (!noise || !actions) return fail(PI_AE_EINVAL, "noise and actions must be non-NULL");
  if (kv->prefix_len > 0 && (!kv->k || !kv->v)) return fail(PI_AE_EINVAL, "prefix k and v must be non-NULL");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (misaligned(noise) || misaligned(actions) || misaligned(kv->k) || misaligned(kv->v))
    return fail(PI_AE_EINVAL, "k, v, noise and actions must be 16-byte aligned");
  return PI_AE_OK;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

ArgsParams args_for(const Workspace& ws, const pi_ae_prefix_kv* kv, const float* noise, float* actions, int batch) {
  ArgsParams a{};
  a.da = ws.da;
  a.vals.pk = static_cast<const uint16_t*>(kv->k);
  a.vals.pv = static_cast<const uint16_t*>(kv->v);
  a.vals.mask = kv->pad_mask;
  a.vals.noise = noise;
  a.vals.actions = actions;
  a.n_valid = ws.n_valid;
  a.B = batch;
  a.P = kv->prefix_len;
  return a;
}

}  // namespace

// ====================================================================== C ABI
PI_AE_API pi_ae_status pi_ae_prepare_weights(const pi_ae_config* cfg, const pi_ae_weights* w, pi_ae_ctx** out) {
  if (!cfg || !w || !out) return fail(PI_AE_EINVAL, "cfg, w and out must be non-NULL");
  pi_ae_status st = check_config(cfg);
  if (st) return st;
  if ((st = check_weights(cfg, w))) return st;
  pi_ae_ctx* ctx = new (std::nothrow) pi_ae_ctx();
  if (!ctx) return fail(PI_AE_ENOMEM, "host allocation failed");
  ctx->cfg = *cfg;
  ctx->arena.arm_fault_injection();
  try {
    HIP_OR_THROW(hipGetDevice(&ctx->device));
    prepare(ctx, w);
  } catch (const HipError& e) {
    ctx->release();
    delete ctx;
    return fail(e.e == hipErrorOutOfMemory ? PI_AE_ENOMEM : PI_AE_EHIP, e.what);
  } catch (const std::bad_alloc&) {
    ctx->release();
    delete ctx;
    return fail(PI_AE_ENOMEM, "host allocation failed during preparation");
  } catch (...) {
    ctx->release();
    delete ctx;
    return fail(PI_AE_EHIP, "unexpected failure during preparation");
  }
  *out = ctx;
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_sample(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise, float* actions,
                                    int32_t batch, void* stream) {
  pi_ae_status st = check_call(ctx, kv, noise, actions, batch);
  if (st || batch == 0) return st;
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const std::pair<int, int> key(batch, kv->prefix_len);
  auto* g = ctx->graphs.find(key);
  if (!g) {
    hipGraphExec_t exec = nullptr;
    hipError_t e = capture_graph(ctx->cap, [&] { return enqueue(ctx, ctx->ws, batch, kv->prefix_len, ctx->cap, StopAt{}); },
                                 &exec);
    if (e == hipSuccess) e = ctx->graphs.insert(key, exec, &g);
    if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("graph capture failed: ") + hipGetErrorString(e));
  }
  hipError_t e = launch_args(args_for(ctx->ws, kv, noise, actions, batch), s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::launch(g, s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::mark(g, s);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
  return PI_AE_OK;
}

namespace {
// Carves the working memory of one call with batch * chunk_len <= 64 rows out
// of a byte range at `base` (256-byte aligned pieces); returns the bytes used.
// With base == nullptr only the size is computed.
size_t noalloc_layout(int L, int B, int T, int nkb, char* base, Workspace* ws) {
  const size_t Mp = size_t(kNoallocMaxRows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  Workspace w;
  w.h = reinterpret_cast<float*>(take(Mp * kD * 4));
  w.q = reinterpret_cast<uint16_t*>(take(Mp * kH * kHd * 2));
  w.o = reinterpret_cast<uint16_t*>(take(Mp * kH * kHd * 2));
  w.o2 = reinterpret_cast<uint16_t*>(take(Mp * kH * kHd * 2 + Mp * kH * 4 * 4));
  w.m = reinterpret_cast<uint16_t*>(take(Mp * kF * 2));
  w.u = reinterpret_cast<uint16_t*>(take(Mp * kD * 2));
  w.ssq = reinterpret_cast<float*>(take(Mp * (kD / 16) * 4));
  w.rope_cs = reinterpret_cast<float2*>(take(Mp * kRopeHalf * 8));
  w.kbias = reinterpret_cast<float*>(take(size_t(B) * nkb * 32 * 4));
  w.n_valid = reinterpret_cast<int*>(take(size_t(B) * 4));
  w.da = reinterpret_cast<DevArgs*>(take(sizeof(DevArgs)));
  w.kp = reinterpret_cast<uint16_t*>(take(size_t(L) * B * nkb * 8192 * 2));
  w.vp = reinterpret_cast<uint16_t*>(take(size_t(L) * B * nkb * 8192 * 2));
  (void)T;
  if (ws) *ws = w;
  return off;
}
}  // namespace

PI_AE_API pi_ae_status pi_ae_sample_noalloc(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise,
                                            float* actions, int32_t batch, void* stream) {
  pi_ae_status st = check_call(ctx, kv, noise, actions, batch);
  if (st || batch == 0) return st;
  const int T = ctx->cfg.chunk_len, L = ctx->cfg.num_layers, P = kv->prefix_len;
  if (batch * T > kNoallocMaxRows)
    return fail(PI_AE_EINVAL, "sample_noalloc: batch * chunk_len must be at most " + std::to_string(kNoallocMaxRows));
  const int nkb = (P + T + 31) / 32;
  const size_t need = noalloc_layout(L, batch, T, nkb, nullptr, nullptr);
  if (need > kNoallocScratchBytes)
    return fail(PI_AE_EINVAL, "sample_noalloc: this call needs " + std::to_string(need) +
                                  " bytes of working memory; the fixed array holds " +
                                  std::to_string(kNoallocScratchBytes) + " (fewer layers or a shorter prefix)");
  DeviceGuard dg(ctx->device);
  void* base = nullptr;
  hipError_t e = noalloc_scratch(&base);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("sample_noalloc: scratch address: ") + hipGetErrorString(e));
  Workspace ws;
  noalloc_layout(L, batch, T, nkb, static_cast<char*>(base), &ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  e = launch_args(args_for(ws, kv, noise, actions, batch), s);
  if (e == hipSuccess) e = enqueue(ctx, ws, batch, P, s, StopAt{});
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("sample_noalloc: launch failed: ") + hipGetErrorString(e));
  return PI_AE_OK;
}

PI_AE_API void pi_ae_destroy(pi_ae_ctx* ctx) {
  if (!ctx) return;
  {
    DeviceGuard dg(ctx->device);
    ctx->release();  // waits for this context's launched graphs, then frees
  }
  delete ctx;
}

PI_AE_API const char* pi_ae_status_string(int32_t s) {
  switch (s) {
    case PI_AE_OK: return "ok";
    case PI_AE_EINVAL: return "invalid argument";
    case PI_AE_EUNSUPPORTED: return "unsupported shape";
    case PI_AE_ENOMEM: return "out of memory";
    case PI_AE_EHIP: return "HIP runtime error";
    case PI_AE_ESTATE: return "invalid context state";
  }
  return "unknown status";
}

PI_AE_API const char* pi_ae_last_error(void) { return g_last_error.c_str(); }

PI_AE_API pi_ae_status pi_ae_debug_table(pi_ae_ctx* ctx, int32_t which, float* host_out, size_t n_floats) {
  if (!ctx || !host_out) return fail(PI_AE_EINVAL, "ctx and host_out must be non-NULL");
  if (which < 0 || which > 9) return fail(PI_AE_EINVAL, "table index out of range");
  const std::vector<float>& t = ctx->tab[which];
  if (n_floats != t.size())
    return fail(PI_AE_EINVAL, "table " + std::to_string(which) + " has " + std::to_string(t.size()) + " floats");
  std::memcpy(host_out, t.data(), t.size() * 4);
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_debug_host_table(const pi_ae_config* cfg, const pi_ae_weights* w, int32_t which,
                                              float* host_out, size_t n_floats) {
  if (!cfg || !w || !host_out) return fail(PI_AE_EINVAL, "cfg, w and host_out must be non-NULL");
  if (which < 0 || which > 9) return fail(PI_AE_EINVAL, "table index out of range");
  pi_ae_status st = check_config(cfg);
  if (st) return st;
  if ((st = check_weights(cfg, w))) return st;
  try {
    std::vector<float> tab[10];
    compute_tables(*cfg, w, tab);
    if (n_floats != tab[which].size())
      return fail(PI_AE_EINVAL, "table " + std::to_string(which) + " has " + std::to_string(tab[which].size()) + " floats");
    std::memcpy(host_out, tab[which].data(), n_floats * 4);
  } catch (const std::bad_alloc&) {
    return fail(PI_AE_ENOMEM, "host allocation failed");
  }
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_debug_time_phase(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise,
                                              float* actions, int32_t batch, int32_t phase, int32_t chunks,
                                              void* stream, float* avg_us) {
  pi_ae_status st = check_call(ctx, kv, noise, actions, batch);
  if (st) return st;
  if (batch < 1 || phase < 0 || phase > 5 || chunks < 1 || chunks > 1000 || !avg_us)
    return fail(PI_AE_EINVAL, "time_phase: batch >= 1, phase in [0, 5], chunks in [1, 1000], avg_us non-NULL");
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = ctx->cfg.num_layers, S = ctx->cfg.num_steps;
  const int per_chunk = phase == 0 ? S + 1 : S * L;
  std::vector<KernelTiming> tv(size_t(per_chunk) * chunks, KernelTiming{nullptr, nullptr});
  hipError_t e = hipSuccess;
  for (auto& t : tv) {
    if (e == hipSuccess) e = hipEventCreate(&t.start);
    if (e == hipSuccess) e = hipEventCreate(&t.stop);
  }
  for (int c = 0; c < chunks && e == hipSuccess; ++c) {
    e = launch_args(args_for(ctx->ws, kv, noise, actions, batch), s);
    if (e == hipSuccess) e = enqueue(ctx, ctx->ws, batch, kv->prefix_len, s, StopAt{}, phase, &tv[size_t(c) * per_chunk]);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  double sum_ms = 0.0;
  for (auto& t : tv) {
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    sum_ms += ms;
  }
  for (auto& t : tv) {
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("time_phase failed: ") + hipGetErrorString(e));
  *avg_us = float(sum_ms * 1000.0 / double(tv.size()));
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_debug_probe(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise,
                                         int32_t batch, int32_t step, int32_t layer, int32_t phase, int32_t which,
                                         void* host_out, size_t n_bytes) {
  if (!ctx) return fail(PI_AE_EINVAL, "ctx is NULL");
  float* actions = nullptr;
  pi_ae_status st = PI_AE_OK;
  if (batch < 1 || batch > ctx->cfg.max_batch) return fail(PI_AE_EINVAL, "probe needs batch in [1, max_batch]");
  if (step < 0 || step > ctx->cfg.num_steps || layer < 0 || layer >= ctx->cfg.num_layers || phase < 0 || phase > 5)
    return fail(PI_AE_EINVAL, "probe position out of range");
  const int T = ctx->cfg.chunk_len, M = batch * T;
  size_t need = 0;
  switch (which) {
    case 0: need = size_t(M) * kD * 4; break;
    case 1: need = size_t(M) * kH * kHd * 2; break;
    case 2: case 3: need = size_t(M) * kHd * 2; break;
    case 4: need = size_t(M) * kH * kHd * 2; break;
    case 5: need = size_t(M) * kF * 2; break;
    case 6: need = size_t(M) * kA * 4; break;
    case 7: need = size_t(M) * kH * kHd * 2; break;
    case 8: need = size_t(M) * kH * 4 * 4; break;
    default: return fail(PI_AE_EINVAL, "probe 'which' out of range");
  }
  if (!host_out || n_bytes != need) return fail(PI_AE_EINVAL, "probe output size must be " + std::to_string(need));
  DeviceGuard dg(ctx->device);
  if (hipMalloc(&actions, size_t(M) * kA * 4) != hipSuccess) return fail(PI_AE_ENOMEM, "probe scratch");
  if ((st = check_call(ctx, kv, noise, actions, batch))) {
    (void)hipFree(actions);
    return st;
  }
  StopAt stop;
  stop.step = step;
  stop.layer = layer;
  stop.phase = phase;
  hipError_t e = launch_args(args_for(ctx->ws, kv, noise, actions, batch), nullptr);
  if (e == hipSuccess) e = enqueue(ctx, ctx->ws, batch, kv->prefix_len, nullptr, stop);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  std::vector<uint16_t> buf;
  if (e == hipSuccess) {
    if (which == 0) {
      e = hipMemcpy(host_out, ctx->ws.h, need, hipMemcpyDeviceToHost);
    } else if (which == 6) {
      e = hipMemcpy(host_out, actions, need, hipMemcpyDeviceToHost);
    } else if (which == 1) {
      e = hipMemcpy(host_out, ctx->ws.q, need, hipMemcpyDeviceToHost);
    } else if (which == 8) {
      e = hipMemcpy(host_out, attn_row_stats(ctx->ws.o2, M), need, hipMemcpyDeviceToHost);
    } else if (which == 2 || which == 3) {
      // suffix keys of layer `layer` from the packed K / V (see kpack_index / vpack_index)
      const int P = kv->prefix_len, nkb = (P + T + 31) / 32;
      const size_t n = size_t(batch) * nkb * 8192;
      buf.resize(n);
      const uint16_t* src = (which == 2 ? ctx->ws.kp : ctx->ws.vp) + size_t(layer) * batch * nkb * 8192;
      e = hipMemcpy(buf.data(), src, n * 2, hipMemcpyDeviceToHost);
      uint16_t* dst = static_cast<uint16_t*>(host_out);
      for (int b = 0; b < batch; ++b)
        for (int t = 0; t < T; ++t)
          for (int d = 0; d < kHd; ++d) {
            const int key = P + t, w32 = key & 31;
            size_t idx;
            if (which == 2) {
              const int lane = (w32 & 15) + 16 * ((d & 31) >> 3);
              idx = ((size_t(b) * nkb + (key >> 5)) * 16 + (w32 >> 4) * 8 + (d >> 5)) * 512 + lane * 8 + (d & 7);
            } else {
              const int r4 = w32 & 15, lane = (d & 15) + 16 * (r4 >> 2);
              idx = ((size_t(b) * nkb + (key >> 5)) * 16 + (d >> 4)) * 512 + lane * 8 + (w32 >> 4) * 4 + (r4 & 3);
            }
            dst[(size_t(b) * T + t) * kHd + d] = buf[idx];
          }
    } else {
      // fragment-major [Mpad/16][K/32][64][8] -> natural [M][K]
      const int K = which == 5 ? kF : kH * kHd;
      const size_t rows = size_t((M + 15) / 16) * 16;
      buf.resize(rows * K);
      e = hipMemcpy(buf.data(), which == 4 ? ctx->ws.o : which == 7 ? ctx->ws.o2 : ctx->ws.m, buf.size() * 2,
                    hipMemcpyDeviceToHost);
      uint16_t* dst = static_cast<uint16_t*>(host_out);
      for (int r = 0; r < M; ++r)
        for (int k = 0; k < K; ++k) {
          const int lane = (r & 15) + 16 * ((k & 31) >> 3);
          dst[size_t(r) * K + k] = buf[((size_t(r >> 4) * (K / 32) + (k >> 5)) * 64 + lane) * 8 + (k & 7)];
        }
    }
  }
  (void)hipFree(actions);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("probe failed: ") + hipGetErrorString(e));
  return PI_AE_OK;
}

// ====================================================================== VLM prefill
struct pi_ae_vlm {
  pi_ae_vlm_config cfg{};
  int device = 0;
  bool broken = false;
  DeviceArena arena;
  // prepared weights (device, swizzled; the last layer has only QKV)
  uint16_t *w_qkv = nullptr, *w_o = nullptr, *w_gu = nullptr, *w_d = nullptr;
  float *attn_s1 = nullptr, *ffn_s1 = nullptr;  // norm scales gamma [L][2048]
  float *zero_qkv = nullptr, *zero_gu = nullptr, *ones = nullptr;
  double* inv_freq = nullptr;
  // workspaces
  float *h = nullptr, *ssq = nullptr, *kbias = nullptr;
  uint16_t *u = nullptr, *q = nullptr, *o = nullptr, *m = nullptr, *kp = nullptr, *vp = nullptr;
  float2* rope_cs = nullptr;
  uint16_t *k_cache = nullptr, *v_cache = nullptr;  // [L][B][P][256] of the last call
  float* part = nullptr;  // split-K partial tiles, up to kVlmMaxSplit x Mpad x 2560
  int Mpad = 0, nkb_max = 0;
  hipStream_t cap = nullptr;
  GraphCache<std::pair<int, int>> graphs;

  template <class T>
  T* dalloc(size_t n) {
    return arena.alloc<T>(n);
  }
  void release() {
    graphs.clear();
    arena.release();
    if (cap) (void)hipStreamDestroy(cap);
    cap = nullptr;
  }
};

namespace {

// K splits of a tiled VLM GEMM (powers of two, at most kVlmMaxSplit, each K
// range a multiple of 256): split while the tiles fill less than half of the
// 256 CUs, or less than all of them while each K range stays >= 4096.  At one
// view (256 rows) the O and down projections have only 64 tiles of 128 x 64,
// QKV 80.  Measured: splitting a K = 2048 GEMM that already has 224 tiles,
// or targeting 512 workgroups, is slower (the partial tiles' extra traffic
// and the second kernel outweigh the parallelism).
constexpr int kVlmMaxSplit = 8;
int vlm_ksplit(int M, int ncols, int bn, int K) {
  const int wgs = (ncols / bn) * ((M + 127) / 128);
  int S = 1;
  while (S < kVlmMaxSplit && K % (256 * S * 2) == 0 &&
         (wgs * S < 128 || (wgs * S < 256 && K / (2 * S) >= 4096)))
    S *= 2;
  return S;
}

pi_ae_status vlm_check_config(const pi_ae_vlm_config* c) {
  if (c->width != kVD || c->mlp_dim != kVF || c->num_heads != kH || c->num_kv_heads != 1 || c->head_dim != kHd)
    return fail(PI_AE_EUNSUPPORTED, "the VLM kernels implement width 2048, mlp_dim 16384, 8 heads x 256, one KV head");
  if (c->num_layers < 1 || c->num_layers > 64) return fail(PI_AE_EINVAL, "num_layers must be in [1, 64]");
  if (c->max_batch < 1 || c->max_prefix_len < 1 || c->max_prefix_len > 4096)
    return fail(PI_AE_EINVAL, "max_batch >= 1 and max_prefix_len in [1, 4096]");
  if (!(c->rope_base > 0.f) || !(c->rms_eps > 0.f)) return fail(PI_AE_EINVAL, "rope_base and rms_eps must be > 0");
  return PI_AE_OK;
}

pi_ae_status vlm_check_weights(const pi_ae_vlm_config* c, const pi_ae_vlm_layer_weights* w) {
  if (!w) return fail(PI_AE_EINVAL, "layers is NULL");
  for (int l = 0; l < c->num_layers; ++l) {
    const pi_ae_vlm_layer_weights& L = w[l];
    const bool last = l == c->num_layers - 1;
    if (!L.attn_norm || !L.q || !L.k || !L.v ||
        (!last && (!L.o || !L.ffn_norm || !L.gate || !L.up || !L.down)))
      return fail(PI_AE_EINVAL, "layer " + std::to_string(l) + ": a weight pointer is NULL");
  }
  return PI_AE_OK;
}

void vlm_prepare(pi_ae_vlm* ctx, const pi_ae_vlm_layer_weights* w) {
  const pi_ae_vlm_config& cfg = ctx->cfg;
  const int L = cfg.num_layers;
  const std::vector<int> pq = qkv_perm(), pg = gu_perm(kVF);
  std::vector<int> pid(kVD);
  for (int i = 0; i < kVD; ++i) pid[i] = i;
  const size_t n_qkv = size_t(kNqkv) * kVD, n_o = size_t(kVD) * kH * kHd, n_gu = size_t(kVNgu) * kVD,
               n_d = size_t(kVD) * kVF;
  ctx->w_qkv = ctx->dalloc<uint16_t>(n_qkv * L);
  if (L > 1) {
    ctx->w_o = ctx->dalloc<uint16_t>(n_o * (L - 1));
    ctx->w_gu = ctx->dalloc<uint16_t>(n_gu * (L - 1));
    ctx->w_d = ctx->dalloc<uint16_t>(n_d * (L - 1));
  }
  {
    std::vector<uint16_t> fused(n_gu), sw(n_gu);
    for (int l = 0; l < L; ++l) {
      const pi_ae_vlm_layer_weights& Lw = w[l];
      std::memcpy(fused.data(), Lw.q, sizeof(uint16_t) * kH * kHd * kVD);
      std::memcpy(fused.data() + size_t(kH) * kHd * kVD, Lw.k, sizeof(uint16_t) * kHd * kVD);
      std::memcpy(fused.data() + size_t(kH + 1) * kHd * kVD, Lw.v, sizeof(uint16_t) * kHd * kVD);
      swizzle(fused.data(), kVD, pq, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_qkv + n_qkv * l, sw.data(), n_qkv * 2, hipMemcpyHostToDevice));
      if (l == L - 1) break;
      swizzle(Lw.o, kH * kHd, pid, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_o + n_o * l, sw.data(), n_o * 2, hipMemcpyHostToDevice));
      std::memcpy(fused.data(), Lw.gate, sizeof(uint16_t) * kVF * kVD);
      std::memcpy(fused.data() + size_t(kVF) * kVD, Lw.up, sizeof(uint16_t) * kVF * kVD);
      swizzle(fused.data(), kVD, pg, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_gu + n_gu * l, sw.data(), n_gu * 2, hipMemcpyHostToDevice));
      swizzle(Lw.down, kVF, pid, sw.data());
      HIP_OR_THROW(hipMemcpy(ctx->w_d + n_d * l, sw.data(), n_d * 2, hipMemcpyHostToDevice));
    }
  }
  auto upload = [&](const std::vector<float>& v) {
    float* d = ctx->dalloc<float>(v.size());
    HIP_OR_THROW(hipMemcpy(d, v.data(), v.size() * 4, hipMemcpyHostToDevice));
    return d;
  };
  {
    std::vector<float> as1(size_t(L) * kVD, 1.f), fs1(size_t(L) * kVD, 1.f);
    for (int l = 0; l < L; ++l)
      for (int i = 0; i < kVD; ++i) {
        as1[size_t(l) * kVD + i] = float(bf(w[l].attn_norm[i]));
        if (l < L - 1) fs1[size_t(l) * kVD + i] = float(bf(w[l].ffn_norm[i]));
      }
    ctx->attn_s1 = upload(as1);
    ctx->ffn_s1 = upload(fs1);
    ctx->zero_qkv = upload(std::vector<float>(kNqkv, 0.f));
    ctx->zero_gu = upload(std::vector<float>(kVNgu, 0.f));
    ctx->ones = upload(std::vector<float>(kVD, 1.f));
    std::vector<double> inv(kRopeHalf);
    for (int i = 0; i < kRopeHalf; ++i) inv[i] = std::pow(double(cfg.rope_base), -2.0 * i / kHd);
    ctx->inv_freq = ctx->dalloc<double>(kRopeHalf);
    HIP_OR_THROW(hipMemcpy(ctx->inv_freq, inv.data(), kRopeHalf * 8, hipMemcpyHostToDevice));
  }
  // workspaces (zeroed once: rows past a call's M are read by whole GEMM
  // tiles but never written by it, and must hold finite values)
  const size_t Mmax = size_t(cfg.max_batch) * cfg.max_prefix_len;
  ctx->Mpad = int((Mmax + 255) / 256 * 256);  // whole 256-row tiles of the wide gate/up GEMM
  const size_t Mp = size_t(ctx->Mpad);
  ctx->nkb_max = (cfg.max_prefix_len + 31) / 32;
  const size_t npack = size_t(cfg.max_batch) * ctx->nkb_max * 8192;
  ctx->h = ctx->dalloc<float>(Mp * kVD);
  ctx->u = ctx->dalloc<uint16_t>(Mp * kVD);
  ctx->ssq = ctx->dalloc<float>(Mp * (kVD / 16));
  ctx->q = ctx->dalloc<uint16_t>(Mp * kH * kHd);
  ctx->o = ctx->dalloc<uint16_t>(Mp * kH * kHd);
  ctx->m = ctx->dalloc<uint16_t>(Mp * kVF);
  ctx->kp = ctx->dalloc<uint16_t>(npack);
  ctx->vp = ctx->dalloc<uint16_t>(npack);
  ctx->kbias = ctx->dalloc<float>(size_t(cfg.max_batch) * ctx->nkb_max * 32);
  ctx->rope_cs = ctx->dalloc<float2>(Mp * kRopeHalf);
  const size_t ncache = size_t(L) * Mmax * kHd;
  ctx->k_cache = ctx->dalloc<uint16_t>(ncache);
  ctx->v_cache = ctx->dalloc<uint16_t>(ncache);
  ctx->part = ctx->dalloc<float>(size_t(kVlmMaxSplit) * Mp * kNqkv);
  HIP_OR_THROW(hipMemset(ctx->h, 0, Mp * kVD * 4));
  HIP_OR_THROW(hipMemset(ctx->u, 0, Mp * kVD * 2));
  HIP_OR_THROW(hipMemset(ctx->ssq, 0, Mp * (kVD / 16) * 4));
  HIP_OR_THROW(hipMemset(ctx->q, 0, Mp * kH * kHd * 2));
  HIP_OR_THROW(hipMemset(ctx->o, 0, Mp * kH * kHd * 2));
  HIP_OR_THROW(hipMemset(ctx->m, 0, Mp * kVF * 2));
  HIP_OR_THROW(hipMemset(ctx->kp, 0, npack * 2));
  HIP_OR_THROW(hipMemset(ctx->vp, 0, npack * 2));
  HIP_OR_THROW(hipStreamCreateWithFlags(&ctx->cap, hipStreamNonBlocking));
  HIP_OR_THROW(hipDeviceSynchronize());
}

// Phases of layer l: 1 = QKV (K/V only in the last layer), 2 = attention,
// 3 = O + residual, 4 = gate/up, 5 = down + residual.
hipError_t vlm_launch_phase(pi_ae_vlm* ctx, int B, int P, hipStream_t s, int l, int ph, const KernelTiming* t) {
  const int L = ctx->cfg.num_layers, M = B * P, nkb = (P + 31) / 32;
  const bool last = l == L - 1;
  const size_t n_qkv = size_t(kNqkv) * kVD, n_o = size_t(kVD) * kH * kHd, n_gu = size_t(kVNgu) * kVD,
               n_d = size_t(kVD) * kVF;
  GemmParams g{};
  g.M = M;
  g.eps = ctx->cfg.rms_eps;
  switch (ph) {
    case 1:
      g.w = ctx->w_qkv + n_qkv * l;
      g.a_frag = ctx->u;
      g.ssq = ctx->ssq;
      g.bias = ctx->zero_qkv;
      g.q_out = ctx->q;
      g.rope_cs = ctx->rope_cs;
      g.T = P;
      g.P = 0;
      g.nkb = nkb;
      g.kp = last ? nullptr : ctx->kp;
      g.vp = last ? nullptr : ctx->vp;
      g.k_cache = ctx->k_cache + size_t(l) * M * kHd;
      g.v_cache = ctx->v_cache + size_t(l) * M * kHd;
      return launch_vlm_qkv(g, last, vlm_ksplit(M, last ? 2 * kHd : kNqkv, 64, kVD), ctx->part, s, t);
    case 2: {
      AttnParams a{};
      a.q = ctx->q;
      a.kp = ctx->kp;
      a.vp = ctx->vp;
      a.kbias = ctx->kbias;
      a.o = ctx->o;
      a.B = B;
      a.T = P;
      a.P = 0;
      a.nkb = nkb;
      return launch_vlm_attn(a, s, t);
    }
    case 3:
      g.w = ctx->w_o + n_o * l;
      g.a_frag = ctx->o;
      g.gate = ctx->ones;
      g.h_out = ctx->h;
      g.s1_next = ctx->ffn_s1 + size_t(l) * kVD;
      g.u_out = ctx->u;
      g.ssq_out = ctx->ssq;
      return launch_vlm_o(g, vlm_ksplit(M, kVD, 64, kH * kHd), ctx->part, s, t);
    case 4:
      g.w = ctx->w_gu + n_gu * l;
      g.a_frag = ctx->u;
      g.ssq = ctx->ssq;
      g.bias = ctx->zero_gu;
      g.m_out = ctx->m;
      return launch_vlm_gu(g, s, t);
    case 5:
      g.w = ctx->w_d + n_d * l;
      g.a_frag = ctx->m;
      g.gate = ctx->ones;
      g.h_out = ctx->h;
      g.s1_next = ctx->attn_s1 + size_t(l + 1) * kVD;
      g.u_out = ctx->u;
      g.ssq_out = ctx->ssq;
      return launch_vlm_down(g, vlm_ksplit(M, kVD, 64, kVF), ctx->part, s, t);
  }
  return hipErrorInvalidValue;
}

hipError_t vlm_enqueue(pi_ae_vlm* ctx, int B, int P, hipStream_t s, int timed_phase = -1,
                       const KernelTiming* timing = nullptr) {
  const int L = ctx->cfg.num_layers;
  int n_timed = 0;
  hipError_t e;
  for (int l = 0; l < L; ++l)
    for (int ph = 1; ph <= (l == L - 1 ? 1 : 5); ++ph) {
      const KernelTiming* t = (timing && ph == timed_phase) ? &timing[n_timed++] : nullptr;
      if ((e = vlm_launch_phase(ctx, B, P, s, l, ph, t)) != hipSuccess) return e;
    }
  return hipSuccess;
}

VlmStageParams vlm_stage_for(pi_ae_vlm* ctx, const uint16_t* emb, const uint8_t* mask, int B, int P) {
  VlmStageParams v{};
  v.emb = emb;
  v.mask = mask;
  v.s1 = ctx->attn_s1;
  v.inv_freq = ctx->inv_freq;
  v.h = ctx->h;
  v.u = ctx->u;
  v.ssq = ctx->ssq;
  v.rope_cs = ctx->rope_cs;
  v.kbias = ctx->kbias;
  v.B = B;
  v.P = P;
  v.nkb = (P + 31) / 32;
  return v;
}

pi_ae_status vlm_check_call(pi_ae_vlm* ctx, const uint16_t* emb, int32_t batch, int32_t P) {
  if (!ctx) return fail(PI_AE_EINVAL, "ctx is NULL");
  if (ctx->broken) return fail(PI_AE_ESTATE, "context is unusable after an earlier failure");
  if (!emb) return fail(PI_AE_EINVAL, "prefix_emb is NULL");
  if ((reinterpret_cast<uintptr_t>(emb) & 15u) != 0) return fail(PI_AE_EINVAL, "prefix_emb must be 16-byte aligned");
  if (batch < 1 || batch > ctx->cfg.max_batch)
    return fail(PI_AE_EINVAL, "batch " + std::to_string(batch) + " outside [1, max_batch]");
  if (P < 1 || P > ctx->cfg.max_prefix_len)
    return fail(PI_AE_EINVAL, "prefix_len " + std::to_string(P) + " outside [1, max_prefix_len]");
  return PI_AE_OK;
}

}  // namespace

PI_AE_API pi_ae_status pi_ae_vlm_prepare(const pi_ae_vlm_config* cfg, const pi_ae_vlm_layer_weights* layers,
                                         pi_ae_vlm** out) {
  if (!cfg || !layers || !out) return fail(PI_AE_EINVAL, "cfg, layers and out must be non-NULL");
  pi_ae_status st = vlm_check_config(cfg);
  if (st) return st;
  if ((st = vlm_check_weights(cfg, layers))) return st;
  pi_ae_vlm* ctx = new (std::nothrow) pi_ae_vlm();
  if (!ctx) return fail(PI_AE_ENOMEM, "host allocation failed");
  ctx->cfg = *cfg;
  ctx->arena.arm_fault_injection();
  try {
    HIP_OR_THROW(hipGetDevice(&ctx->device));
    vlm_prepare(ctx, layers);
  } catch (const HipError& e) {
    ctx->release();
    delete ctx;
    return fail(e.e == hipErrorOutOfMemory ? PI_AE_ENOMEM : PI_AE_EHIP, e.what);
  } catch (const std::bad_alloc&) {
    ctx->release();
    delete ctx;
    return fail(PI_AE_ENOMEM, "host allocation failed during preparation");
  } catch (...) {
    ctx->release();
    delete ctx;
    return fail(PI_AE_EHIP, "unexpected failure during preparation");
  }
  *out = ctx;
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_vlm_prefill(pi_ae_vlm* ctx, const uint16_t* prefix_emb, const uint8_t* pad_mask,
                                         int32_t batch, int32_t prefix_len, pi_ae_prefix_kv* kv_out, void* stream) {
  pi_ae_status st = vlm_check_call(ctx, prefix_emb, batch, prefix_len);
  if (st) return st;
  if (!kv_out) return fail(PI_AE_EINVAL, "kv_out is NULL");
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const std::pair<int, int> key(batch, prefix_len);
  auto* g = ctx->graphs.find(key);
  if (!g) {
    hipGraphExec_t exec = nullptr;
    hipError_t e = capture_graph(ctx->cap, [&] { return vlm_enqueue(ctx, batch, prefix_len, ctx->cap); }, &exec);
    if (e == hipSuccess) e = ctx->graphs.insert(key, exec, &g);
    if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("graph capture failed: ") + hipGetErrorString(e));
  }
  hipError_t e = launch_vlm_stage(vlm_stage_for(ctx, prefix_emb, pad_mask, batch, prefix_len), s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::launch(g, s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::mark(g, s);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
  kv_out->k = ctx->k_cache;
  kv_out->v = ctx->v_cache;
  kv_out->pad_mask = pad_mask;
  kv_out->prefix_len = prefix_len;
  return PI_AE_OK;
}

PI_AE_API void pi_ae_vlm_destroy(pi_ae_vlm* ctx) {
  if (!ctx) return;
  {
    DeviceGuard dg(ctx->device);
    ctx->release();  // waits for its own launched graphs, then frees
  }
  delete ctx;
}

PI_AE_API pi_ae_status pi_ae_vlm_debug_time_phase(pi_ae_vlm* ctx, const uint16_t* prefix_emb, const uint8_t* pad_mask,
                                                  int32_t batch, int32_t prefix_len, int32_t phase, int32_t reps,
                                                  void* stream, float* avg_us) {
  pi_ae_status st = vlm_check_call(ctx, prefix_emb, batch, prefix_len);
  if (st) return st;
  const int L = ctx->cfg.num_layers;
  if (phase < 1 || phase > 5 || reps < 1 || reps > 1000 || !avg_us || (phase > 1 && L < 2))
    return fail(PI_AE_EINVAL, "time_phase: phase in [1, 5] (2..5 need 2 layers), reps in [1, 1000], avg_us non-NULL");
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int per = phase == 1 ? L : L - 1;
  std::vector<KernelTiming> tv(size_t(per) * reps, KernelTiming{nullptr, nullptr});
  hipError_t e = hipSuccess;
  for (auto& t : tv) {
    if (e == hipSuccess) e = hipEventCreate(&t.start);
    if (e == hipSuccess) e = hipEventCreate(&t.stop);
  }
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    e = launch_vlm_stage(vlm_stage_for(ctx, prefix_emb, pad_mask, batch, prefix_len), s);
    if (e == hipSuccess) e = vlm_enqueue(ctx, batch, prefix_len, s, phase, &tv[size_t(r) * per]);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  double sum_ms = 0.0;
  for (auto& t : tv) {
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    sum_ms += ms;
  }
  for (auto& t : tv) {
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("time_phase failed: ") + hipGetErrorString(e));
  *avg_us = float(sum_ms * 1000.0 / double(tv.size()));
  return PI_AE_OK;
}

// ====================================================================== pipeline
struct pi_ae_pipeline {
  pi_ae_vlm* vlm = nullptr;
  pi_ae_ctx* ctx = nullptr;
  GraphCache<std::pair<int, int>> graphs;
  void release() { graphs.clear(); }
};

PI_AE_API pi_ae_status pi_ae_pipeline_create(pi_ae_vlm* vlm, pi_ae_ctx* expert, pi_ae_pipeline** out) {
  if (!vlm || !expert || !out) return fail(PI_AE_EINVAL, "vlm, expert and out must be non-NULL");
  if (vlm->cfg.num_layers != expert->cfg.num_layers)
    return fail(PI_AE_EINVAL, "the VLM has " + std::to_string(vlm->cfg.num_layers) + " layers, the expert " +
                                  std::to_string(expert->cfg.num_layers));
  if (vlm->device != expert->device) return fail(PI_AE_EINVAL, "the two contexts live on different devices");
  pi_ae_pipeline* p = new (std::nothrow) pi_ae_pipeline();
  if (!p) return fail(PI_AE_ENOMEM, "host allocation failed");
  p->vlm = vlm;
  p->ctx = expert;
  *out = p;
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_pipeline_run(pi_ae_pipeline* pipe, const uint16_t* prefix_emb, const uint8_t* pad_mask,
                                          const float* noise, float* actions, int32_t batch, int32_t prefix_len,
                                          void* stream) {
  if (!pipe) return fail(PI_AE_EINVAL, "pipe is NULL");
  pi_ae_vlm* vlm = pipe->vlm;
  pi_ae_ctx* ctx = pipe->ctx;
  pi_ae_status st = vlm_check_call(vlm, prefix_emb, batch, prefix_len);
  if (st) return st;
  pi_ae_prefix_kv kv{vlm->k_cache, vlm->v_cache, pad_mask, prefix_len};
  if ((st = check_call(ctx, &kv, noise, actions, batch))) return st;
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const std::pair<int, int> key(batch, prefix_len);
  auto* g = pipe->graphs.find(key);
  if (!g) {
    hipGraphExec_t exec = nullptr;
    hipError_t e = capture_graph(ctx->cap, [&] {
      hipError_t e2 = vlm_enqueue(vlm, batch, prefix_len, ctx->cap);
      if (e2 == hipSuccess) e2 = enqueue(ctx, ctx->ws, batch, prefix_len, ctx->cap, StopAt{});
      return e2;
    }, &exec);
    if (e == hipSuccess) e = pipe->graphs.insert(key, exec, &g);
    if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("graph capture failed: ") + hipGetErrorString(e));
  }
  hipError_t e = launch_vlm_stage(vlm_stage_for(vlm, prefix_emb, pad_mask, batch, prefix_len), s);
  if (e == hipSuccess) e = launch_args(args_for(ctx->ws, &kv, noise, actions, batch), s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::launch(g, s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::mark(g, s);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
  return PI_AE_OK;
}

PI_AE_API void pi_ae_pipeline_destroy(pi_ae_pipeline* pipe) {
  if (!pipe) return;
  {
    DeviceGuard dg(pipe->ctx->device);
    pipe->release();  // waits for its own launched graphs, then frees
  }
  delete pipe;
}

// ====================================================================== vision encoder
struct pi_ae_vision {
  pi_ae_vision_config cfg{};
  int device = 0;
  bool broken = false;
  DeviceArena arena;
  // prepared weights (device, swizzled, K padded with zero columns)
  uint16_t *w_patch = nullptr, *w_qkv = nullptr, *w_o = nullptr, *w_fc1 = nullptr, *w_fc2 = nullptr,
           *w_proj = nullptr;
  float *b_patch = nullptr, *pos = nullptr, *b_qkv = nullptr, *b_o = nullptr, *b_fc1 = nullptr, *b_fc2 = nullptr,
        *b_proj = nullptr, *ln1_w = nullptr, *ln1_b = nullptr, *ln2_w = nullptr, *ln2_b = nullptr,
        *post_w = nullptr, *post_b = nullptr;
  // workspaces
  uint16_t *apatch = nullptr, *u = nullptr, *qkv = nullptr, *o = nullptr, *m = nullptr;
  float *h = nullptr, *part = nullptr;
  int Mpad = 0;
  hipStream_t cap = nullptr;
  GraphCache<int> graphs;

  template <class T>
  T* dalloc(size_t n) {
    return arena.alloc<T>(n);
  }
  void release() {
    graphs.clear();
    arena.release();
    if (cap) (void)hipStreamDestroy(cap);
    cap = nullptr;
  }
};

namespace {

// K split of a vision GEMM (128 x 64 tiles): the largest of 2, 3, 6 whose K
// ranges are whole 256-wide blocks of at least 768 and whose launch stays
// within one workgroup per CU.  Only fc2 (K 4608) qualifies: 6 ranges at one
// view, 3 at two, 2 at three.  Measured at one view: fc2 22.0 -> 16.5 us with
// 6 ranges; splitting the K = 1280 GEMMs into five 256-wide ranges, or fc2
// at three views beyond 2, was slower (the partial tiles and the reduce cost
// more than the shorter K loop saves).
constexpr int kVisMaxSplit = 6;
// K ranges of the O projection (K 1280 = 5 x 256): five when they still fit
// in one round of workgroups, else one
int vis_osplit(int M) { return (kSD / 64) * ((M + 127) / 128) * 5 <= 256 ? 5 : 1; }
unsigned row_tiles128(int M) { return unsigned((M + 127) / 128); }
int vis_ksplit(int M, int ncols, int K) {
  if (ncols > kSD) return 1;  // the partial-tile buffer holds kVisMaxSplit x Mpad x 1152
  const int wgs = (ncols / 64) * ((M + 127) / 128);
  int S = 1;
  for (int c : {2, 3, 6})
    if (K % (256 * c) == 0 && K / c >= 768 && wgs * c <= 256) S = c;
  return S;
}

pi_ae_status vis_check_config(const pi_ae_vision_config* c) {
  if (c->width != kSD || c->mlp_dim != kSF || c->num_heads != kSH || c->head_dim != kSHd || c->patch != kSPatch ||
      c->image != kSImg || c->out_width != kSOut)
    return fail(PI_AE_EUNSUPPORTED,
                "the vision kernels implement width 1152, mlp_dim 4304, 16 heads x 72, patch 14, image 224, out 2048");
  if (c->num_layers < 1 || c->num_layers > 64) return fail(PI_AE_EINVAL, "num_layers must be in [1, 64]");
  if (c->max_views < 1 || c->max_views > 64) return fail(PI_AE_EINVAL, "max_views must be in [1, 64]");
  if (!(c->ln_eps > 0.f)) return fail(PI_AE_EINVAL, "ln_eps must be > 0");
  return PI_AE_OK;
}

pi_ae_status vis_check_weights(const pi_ae_vision_config* c, const pi_ae_vision_weights* w) {
  if (!w->patch_w || !w->patch_b || !w->pos || !w->layers || !w->post_ln_w || !w->post_ln_b || !w->proj_w || !w->proj_b)
    return fail(PI_AE_EINVAL, "a vision weight pointer is NULL");
  for (int l = 0; l < c->num_layers; ++l) {
    const pi_ae_vision_layer_weights& L = w->layers[l];
    const uint16_t* ps[] = {L.ln1_w, L.ln1_b, L.q_w, L.q_b, L.k_w, L.k_b, L.v_w, L.v_b, L.o_w, L.o_b,
                            L.ln2_w, L.ln2_b, L.fc1_w, L.fc1_b, L.fc2_w, L.fc2_b};
    for (const uint16_t* q : ps)
      if (!q) return fail(PI_AE_EINVAL, "vision layer " + std::to_string(l) + ": a weight pointer is NULL");
  }
  return PI_AE_OK;
}

// W [N][K] -> [Np][Kp] with zero rows / columns past N / K
std::vector<uint16_t> pad2(const uint16_t* W, int N, int K, int Np, int Kp) {
  std::vector<uint16_t> out(size_t(Np) * Kp, 0);
  for (int n = 0; n < N; ++n) std::memcpy(out.data() + size_t(n) * Kp, W + size_t(n) * K, size_t(K) * 2);
  return out;
}

std::vector<float> to_f32(const uint16_t* b, int n, int npad) {
  std::vector<float> out(npad, 0.f);
  for (int i = 0; i < n; ++i) out[i] = float(bf(b[i]));
  return out;
}

void vis_prepare(pi_ae_vision* ctx, const pi_ae_vision_weights* w) {
  const int L = ctx->cfg.num_layers;
  auto ident = [](int n) {
    std::vector<int> p(n);
    for (int i = 0; i < n; ++i) p[i] = i;
    return p;
  };
  auto upload16 = [&](const std::vector<uint16_t>& v, uint16_t* dst) {
    HIP_OR_THROW(hipMemcpy(dst, v.data(), v.size() * 2, hipMemcpyHostToDevice));
  };
  auto swz = [&](const uint16_t* W, int N, int K, int Np, int Kp, uint16_t* dst) {
    const std::vector<uint16_t> padded = pad2(W, N, K, Np, Kp);
    std::vector<uint16_t> sw(padded.size());
    swizzle(padded.data(), Kp, ident(Np), sw.data());
    upload16(sw, dst);
  };
  const int kpv = kSC * kSPatch * kSPatch;  // 588
  const size_t n_qkv = size_t(3 * kSD) * kSKp, n_o = size_t(kSD) * kSKp, n_fc1 = size_t(kSFn) * kSKp,
               n_fc2 = size_t(kSD) * kSFk;
  ctx->w_patch = ctx->dalloc<uint16_t>(size_t(kSD) * kSKpatch);
  swz(w->patch_w, kSD, kpv, kSD, kSKpatch, ctx->w_patch);
  ctx->w_qkv = ctx->dalloc<uint16_t>(n_qkv * L);
  ctx->w_o = ctx->dalloc<uint16_t>(n_o * L);
  ctx->w_fc1 = ctx->dalloc<uint16_t>(n_fc1 * L);
  ctx->w_fc2 = ctx->dalloc<uint16_t>(n_fc2 * L);
  std::vector<float> bqkv(size_t(L) * 3 * kSD), bo(size_t(L) * kSD), bfc1(size_t(L) * kSFn, 0.f), bfc2(size_t(L) * kSD),
      l1w(size_t(L) * kSD), l1b(size_t(L) * kSD), l2w(size_t(L) * kSD), l2b(size_t(L) * kSD);
  for (int l = 0; l < L; ++l) {
    const pi_ae_vision_layer_weights& Lw = w->layers[l];
    std::vector<uint16_t> fused(size_t(3 * kSD) * kSD);
    std::memcpy(fused.data(), Lw.q_w, size_t(kSD) * kSD * 2);
    std::memcpy(fused.data() + size_t(kSD) * kSD, Lw.k_w, size_t(kSD) * kSD * 2);
    std::memcpy(fused.data() + size_t(2 * kSD) * kSD, Lw.v_w, size_t(kSD) * kSD * 2);
    swz(fused.data(), 3 * kSD, kSD, 3 * kSD, kSKp, ctx->w_qkv + n_qkv * l);
    swz(Lw.o_w, kSD, kSD, kSD, kSKp, ctx->w_o + n_o * l);
    swz(Lw.fc1_w, kSF, kSD, kSFn, kSKp, ctx->w_fc1 + n_fc1 * l);
    swz(Lw.fc2_w, kSD, kSF, kSD, kSFk, ctx->w_fc2 + n_fc2 * l);
    for (int i = 0; i < kSD; ++i) {
      bqkv[size_t(l) * 3 * kSD + i] = float(bf(Lw.q_b[i]));
      bqkv[size_t(l) * 3 * kSD + kSD + i] = float(bf(Lw.k_b[i]));
      bqkv[size_t(l) * 3 * kSD + 2 * kSD + i] = float(bf(Lw.v_b[i]));
      bo[size_t(l) * kSD + i] = float(bf(Lw.o_b[i]));
      bfc2[size_t(l) * kSD + i] = float(bf(Lw.fc2_b[i]));
      l1w[size_t(l) * kSD + i] = float(bf(Lw.ln1_w[i]));
      l1b[size_t(l) * kSD + i] = float(bf(Lw.ln1_b[i]));
      l2w[size_t(l) * kSD + i] = float(bf(Lw.ln2_w[i]));
      l2b[size_t(l) * kSD + i] = float(bf(Lw.ln2_b[i]));
    }
    for (int i = 0; i < kSF; ++i) bfc1[size_t(l) * kSFn + i] = float(bf(Lw.fc1_b[i]));
  }
  ctx->w_proj = ctx->dalloc<uint16_t>(size_t(kSOut) * kSKp);
  swz(w->proj_w, kSOut, kSD, kSOut, kSKp, ctx->w_proj);
  auto upload = [&](const std::vector<float>& v) {
    float* d = ctx->dalloc<float>(v.size());
    HIP_OR_THROW(hipMemcpy(d, v.data(), v.size() * 4, hipMemcpyHostToDevice));
    return d;
  };
  ctx->b_patch = upload(to_f32(w->patch_b, kSD, kSD));
  ctx->pos = upload(to_f32(w->pos, kSTok * kSD, kSTok * kSD));
  ctx->b_qkv = upload(bqkv);
  ctx->b_o = upload(bo);
  ctx->b_fc1 = upload(bfc1);
  ctx->b_fc2 = upload(bfc2);
  ctx->ln1_w = upload(l1w);
  ctx->ln1_b = upload(l1b);
  ctx->ln2_w = upload(l2w);
  ctx->ln2_b = upload(l2b);
  ctx->post_w = upload(to_f32(w->post_ln_w, kSD, kSD));
  ctx->post_b = upload(to_f32(w->post_ln_b, kSD, kSD));
  ctx->b_proj = upload(to_f32(w->proj_b, kSOut, kSOut));
  // workspaces; zeroed once: padded operand columns are never written
  const size_t Mmax = size_t(ctx->cfg.max_views) * kSTok;
  ctx->Mpad = int((Mmax + 255) / 256 * 256);
  const size_t Mp = size_t(ctx->Mpad);
  ctx->apatch = ctx->dalloc<uint16_t>(Mp * kSKpatch);
  ctx->h = ctx->dalloc<float>(Mp * kSD);
  ctx->u = ctx->dalloc<uint16_t>(Mp * kSKp);
  ctx->qkv = ctx->dalloc<uint16_t>(Mp * 3 * kSD);
  ctx->o = ctx->dalloc<uint16_t>(Mp * kSKp);
  ctx->m = ctx->dalloc<uint16_t>(Mp * kSFk);
  ctx->part = ctx->dalloc<float>(size_t(kVisMaxSplit) * Mp * kSD);
  HIP_OR_THROW(hipMemset(ctx->apatch, 0, Mp * kSKpatch * 2));
  HIP_OR_THROW(hipMemset(ctx->h, 0, Mp * kSD * 4));
  HIP_OR_THROW(hipMemset(ctx->u, 0, Mp * kSKp * 2));
  HIP_OR_THROW(hipMemset(ctx->qkv, 0, Mp * 3 * kSD * 2));
  HIP_OR_THROW(hipMemset(ctx->o, 0, Mp * kSKp * 2));
  HIP_OR_THROW(hipMemset(ctx->m, 0, Mp * kSFk * 2));
  HIP_OR_THROW(hipStreamCreateWithFlags(&ctx->cap, hipStreamNonBlocking));
  HIP_OR_THROW(hipDeviceSynchronize());
}

// Phases (numbering of pi_ae_vision_debug_time_phase): 0 patch embedding,
// per layer 1 LayerNorm (twice), 2 QKV, 3 attention, 4 O, 5 fc1, 6 fc2; 7
// projector.  The graph holds the patch GEMM through the final LayerNorm;
// the patch vectors (before it) and the projector (after it) take the call's
// pointers.
hipError_t vis_enqueue_layers(pi_ae_vision* ctx, int V, hipStream_t s, int timed, const KernelTiming* tv,
                              int* n_timed) {
  const int L = ctx->cfg.num_layers, M = V * kSTok;
  auto tm = [&](int ph) { return (tv && ph == timed) ? &tv[(*n_timed)++] : nullptr; };
  hipError_t e;
  GemmParams g{};
  g.M = M;
  g.w = ctx->w_patch;
  g.a_frag = ctx->apatch;
  g.bias = ctx->b_patch;
  g.aux = ctx->pos;
  g.h_out = ctx->h;
  if ((e = launch_vis_gemm(0, g, vis_ksplit(M, kSD, kSKpatch), ctx->part, s, tm(0))) != hipSuccess) return e;
  // every LayerNorm but layer 0's first one ends the residual GEMM before it
  // (O, fc2): the raw K-split GEMM, then one kernel that sums its ranges,
  // adds bias and residual and normalises the whole row
  VisLnParams ln{};
  ln.h = ctx->h;
  ln.u = ctx->u;
  ln.eps = ctx->cfg.ln_eps;
  ln.M = M;
  ln.part = ctx->part;
  ln.Mp = int(row_tiles128(M)) * 128;
  ln.w = ctx->ln1_w;
  ln.b = ctx->ln1_b;
  {
    const KernelTiming* t = tm(1);
    if (t && (e = hipEventRecord(t->start, s)) != hipSuccess) return e;
    if ((e = launch_vis_ln(ln, s)) != hipSuccess) return e;
    if (t && (e = hipEventRecord(t->stop, s)) != hipSuccess) return e;
  }
  const int So = vis_osplit(M), Sf = vis_ksplit(M, kSD, kSFk);
  // the raw GEMM and the residual + LayerNorm kernel, timed as one phase
  auto res_ln = [&](int which, const GemmParams& g, int S, const float* bias, const float* w, const float* b,
                    const KernelTiming* t) {
    const KernelTiming t0{t ? t->start : nullptr, nullptr}, t1{nullptr, t ? t->stop : nullptr};
    hipError_t r = launch_vis_gemm_raw(which, g, S, ctx->part, s, t ? &t0 : nullptr);
    if (r != hipSuccess) return r;
    VisLnParams q = ln;
    q.S = S;
    q.bias = bias;
    q.w = w;
    q.b = b;
    return launch_vis_res_ln(q, s, t ? &t1 : nullptr);
  };
  const size_t n_qkv = size_t(3 * kSD) * kSKp, n_o = size_t(kSD) * kSKp, n_fc1 = size_t(kSFn) * kSKp,
               n_fc2 = size_t(kSD) * kSFk;
  for (int l = 0; l < L; ++l) {
    GemmParams q{};
    q.M = M;
    q.w = ctx->w_qkv + n_qkv * l;
    q.a_frag = ctx->u;
    q.bias = ctx->b_qkv + size_t(l) * 3 * kSD;
    q.q_out = ctx->qkv;
    if ((e = launch_vis_gemm(1, q, vis_ksplit(M, 3 * kSD, kSKp), ctx->part, s, tm(2))) != hipSuccess) return e;
    VisAttnParams a{};
    a.qkv = ctx->qkv;
    a.o = ctx->o;
    a.V = V;
    if ((e = launch_vis_attn(a, s, tm(3))) != hipSuccess) return e;
    GemmParams og{};
    og.M = M;
    og.w = ctx->w_o + n_o * l;
    og.a_frag = ctx->o;
    if ((e = res_ln(2, og, So, ctx->b_o + size_t(l) * kSD, ctx->ln2_w + size_t(l) * kSD, ctx->ln2_b + size_t(l) * kSD,
                    tm(4))) != hipSuccess)
      return e;
    GemmParams f1{};
    f1.M = M;
    f1.w = ctx->w_fc1 + n_fc1 * l;
    f1.a_frag = ctx->u;
    f1.bias = ctx->b_fc1 + size_t(l) * kSFn;
    f1.m_out = ctx->m;
    if ((e = launch_vis_gemm(3, f1, vis_ksplit(M, kSFn, kSKp), ctx->part, s, tm(5))) != hipSuccess) return e;
    GemmParams f2{};
    f2.M = M;
    f2.w = ctx->w_fc2 + n_fc2 * l;
    f2.a_frag = ctx->m;
    // the next layer's first LayerNorm, or the final one before the projector
    const bool last = l + 1 == L;
    const float* nw = last ? ctx->post_w : ctx->ln1_w + size_t(l + 1) * kSD;
    const float* nb = last ? ctx->post_b : ctx->ln1_b + size_t(l + 1) * kSD;
    if ((e = res_ln(4, f2, Sf, ctx->b_fc2 + size_t(l) * kSD, nw, nb, tm(6))) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t vis_projector(pi_ae_vision* ctx, int V, uint16_t* tokens, hipStream_t s, const KernelTiming* t) {
  GemmParams g{};
  g.M = V * kSTok;
  g.w = ctx->w_proj;
  g.a_frag = ctx->u;
  g.bias = ctx->b_proj;
  g.q_out = tokens;
  return launch_vis_gemm(5, g, vis_ksplit(g.M, kSOut, kSKp), ctx->part, s, t);
}

pi_ae_status vis_check_call(pi_ae_vision* ctx, const uint16_t* images, int32_t views, const uint16_t* tokens) {
  if (!ctx) return fail(PI_AE_EINVAL, "ctx is NULL");
  if (ctx->broken) return fail(PI_AE_ESTATE, "context is unusable after an earlier failure");
  if (!images || !tokens) return fail(PI_AE_EINVAL, "images and tokens must be non-NULL");
  if (((reinterpret_cast<uintptr_t>(images) | reinterpret_cast<uintptr_t>(tokens)) & 15u) != 0)
    return fail(PI_AE_EINVAL, "images and tokens must be 16-byte aligned");
  if (views < 1 || views > ctx->cfg.max_views)
    return fail(PI_AE_EINVAL, "views " + std::to_string(views) + " outside [1, max_views]");
  return PI_AE_OK;
}

}  // namespace

PI_AE_API pi_ae_status pi_ae_vision_prepare(const pi_ae_vision_config* cfg, const pi_ae_vision_weights* w,
                                            pi_ae_vision** out) {
  if (!cfg || !w || !out) return fail(PI_AE_EINVAL, "cfg, w and out must be non-NULL");
  pi_ae_status st = vis_check_config(cfg);
  if (st) return st;
  if ((st = vis_check_weights(cfg, w))) return st;
  pi_ae_vision* ctx = new (std::nothrow) pi_ae_vision();
  if (!ctx) return fail(PI_AE_ENOMEM, "host allocation failed");
  ctx->cfg = *cfg;
  ctx->arena.arm_fault_injection();
  try {
    HIP_OR_THROW(hipGetDevice(&ctx->device));
    vis_prepare(ctx, w);
  } catch (const HipError& e) {
    ctx->release();
    delete ctx;
    return fail(e.e == hipErrorOutOfMemory ? PI_AE_ENOMEM : PI_AE_EHIP, e.what);
  } catch (const std::bad_alloc&) {
    ctx->release();
    delete ctx;
    return fail(PI_AE_ENOMEM, "host allocation failed during preparation");
  } catch (...) {
    ctx->release();
    delete ctx;
    return fail(PI_AE_EHIP, "unexpected failure during preparation");
  }
  *out = ctx;
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_vision_encode(pi_ae_vision* ctx, const uint16_t* images, int32_t views, uint16_t* tokens,
                                           void* stream) {
  pi_ae_status st = vis_check_call(ctx, images, views, tokens);
  if (st) return st;
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* g = ctx->graphs.find(views);
  if (!g) {
    hipGraphExec_t exec = nullptr;
    hipError_t e = capture_graph(ctx->cap, [&] {
      int n = 0;
      return vis_enqueue_layers(ctx, views, ctx->cap, -1, nullptr, &n);
    }, &exec);
    if (e == hipSuccess) e = ctx->graphs.insert(views, exec, &g);
    if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("graph capture failed: ") + hipGetErrorString(e));
  }
  VisPatchParams pp{images, ctx->apatch, views};
  hipError_t e = launch_vis_patch(pp, s);
  if (e == hipSuccess) e = GraphCache<int>::launch(g, s);
  if (e == hipSuccess) e = vis_projector(ctx, views, tokens, s, nullptr);
  if (e == hipSuccess) e = GraphCache<int>::mark(g, s);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
  return PI_AE_OK;
}

PI_AE_API void pi_ae_vision_destroy(pi_ae_vision* ctx) {
  if (!ctx) return;
  {
    DeviceGuard dg(ctx->device);
    ctx->release();  // waits for its own launched graphs, then frees
  }
  delete ctx;
}

PI_AE_API pi_ae_status pi_ae_vision_debug_time_phase(pi_ae_vision* ctx, const uint16_t* images, int32_t views,
                                                     uint16_t* tokens, int32_t phase, int32_t reps, void* stream,
                                                     float* avg_us) {
  pi_ae_status st = vis_check_call(ctx, images, views, tokens);
  if (st) return st;
  if (phase < 0 || phase > 7 || reps < 1 || reps > 1000 || !avg_us)
    return fail(PI_AE_EINVAL, "time_phase: phase in [0, 7], reps in [1, 1000], avg_us non-NULL");
  DeviceGuard dg(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = ctx->cfg.num_layers;
  const int per = (phase == 0 || phase == 1 || phase == 7) ? 1 : L;  // phase 1: layer 0's first LayerNorm
  std::vector<KernelTiming> tv(size_t(per) * reps, KernelTiming{nullptr, nullptr});
  hipError_t e = hipSuccess;
  for (auto& t : tv) {
    if (e == hipSuccess) e = hipEventCreate(&t.start);
    if (e == hipSuccess) e = hipEventCreate(&t.stop);
  }
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    VisPatchParams pp{images, ctx->apatch, views};
    e = launch_vis_patch(pp, s);
    int n = 0;
    if (e == hipSuccess) e = vis_enqueue_layers(ctx, views, s, phase, &tv[size_t(r) * per], &n);
    if (e == hipSuccess) e = vis_projector(ctx, views, tokens, s, phase == 7 ? &tv[size_t(r) * per] : nullptr);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  double sum_ms = 0.0;
  for (auto& t : tv) {
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    sum_ms += ms;
  }
  for (auto& t : tv) {
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("time_phase failed: ") + hipGetErrorString(e));
  *avg_us = float(sum_ms * 1000.0 / double(tv.size()));
  return PI_AE_OK;
}

// ====================================================================== whole inference
struct pi_ae_inference {
  pi_ae_vision* vis = nullptr;
  pi_ae_vlm* vlm = nullptr;
  pi_ae_ctx* ctx = nullptr;
  uint16_t* prefix = nullptr;  // [max_prefix_len][2048] bf16: the views' tokens, then the prompt's
  uint8_t* mask = nullptr;     // [max_prefix_len]
  GraphCache<std::pair<int, int>> graphs;
  void release() {
    graphs.clear();
    if (prefix) (void)hipFree(prefix);
    if (mask) (void)hipFree(mask);
    prefix = nullptr;
    mask = nullptr;
  }
};

PI_AE_API pi_ae_status pi_ae_inference_create(pi_ae_vision* vision, pi_ae_vlm* vlm, pi_ae_ctx* expert,
                                              pi_ae_inference** out) {
  if (!vision || !vlm || !expert || !out) return fail(PI_AE_EINVAL, "vision, vlm, expert and out must be non-NULL");
  if (vlm->cfg.num_layers != expert->cfg.num_layers)
    return fail(PI_AE_EINVAL, "the VLM and the expert must have the same number of layers");
  if (vision->device != vlm->device || vlm->device != expert->device)
    return fail(PI_AE_EINVAL, "the three contexts live on different devices");
  pi_ae_inference* inf = new (std::nothrow) pi_ae_inference();
  if (!inf) return fail(PI_AE_ENOMEM, "host allocation failed");
  inf->vis = vision;
  inf->vlm = vlm;
  inf->ctx = expert;
  DeviceGuard dg(vlm->device);
  const size_t P = size_t(vlm->cfg.max_prefix_len);
  hipError_t e = hipMalloc(&inf->prefix, P * kSOut * 2);
  if (e == hipSuccess) e = hipMalloc(&inf->mask, P);
  if (e == hipSuccess) e = hipMemset(inf->prefix, 0, P * kSOut * 2);
  if (e != hipSuccess) {
    inf->release();
    delete inf;
    return fail(e == hipErrorOutOfMemory ? PI_AE_ENOMEM : PI_AE_EHIP, std::string("inference buffers: ") + hipGetErrorString(e));
  }
  *out = inf;
  return PI_AE_OK;
}

PI_AE_API pi_ae_status pi_ae_inference_run(pi_ae_inference* inf, const uint16_t* images, int32_t views,
                                           const uint16_t* prompt_emb, int32_t prompt_len, const uint8_t* pad_mask,
                                           const float* noise, float* actions, void* stream) {
  if (!inf) return fail(PI_AE_EINVAL, "inf is NULL");
  pi_ae_status st = vis_check_call(inf->vis, images, views, inf->prefix);
  if (st) return st;
  if (prompt_len < 0 || (prompt_len > 0 && !prompt_emb)) return fail(PI_AE_EINVAL, "prompt_emb / prompt_len");
  const int P = views * kSTok + prompt_len;
  if ((st = vlm_check_call(inf->vlm, inf->prefix, 1, P))) return st;
  pi_ae_prefix_kv kv{inf->vlm->k_cache, inf->vlm->v_cache, inf->mask, P};
  if ((st = check_call(inf->ctx, &kv, noise, actions, 1))) return st;
  DeviceGuard dg(inf->ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const std::pair<int, int> key(views, prompt_len);
  auto* g = inf->graphs.find(key);
  if (!g) {
    hipGraphExec_t exec = nullptr;
    hipStream_t c = inf->ctx->cap;
    hipError_t e = capture_graph(c, [&] {
      int n = 0;
      hipError_t e2 = vis_enqueue_layers(inf->vis, views, c, -1, nullptr, &n);
      if (e2 == hipSuccess) e2 = vis_projector(inf->vis, views, inf->prefix, c, nullptr);
      if (e2 == hipSuccess) e2 = launch_vlm_stage(vlm_stage_for(inf->vlm, inf->prefix, inf->mask, 1, P), c);
      if (e2 == hipSuccess) e2 = vlm_enqueue(inf->vlm, 1, P, c);
      if (e2 == hipSuccess) e2 = enqueue(inf->ctx, inf->ctx->ws, 1, P, c, StopAt{});
      return e2;
    }, &exec);
    if (e == hipSuccess) e = inf->graphs.insert(key, exec, &g);
    if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("graph capture failed: ") + hipGetErrorString(e));
  }
  hipError_t e = hipSuccess;
  if (prompt_len > 0)
    e = hipMemcpyAsync(inf->prefix + size_t(views) * kSTok * kSOut, prompt_emb, size_t(prompt_len) * kSOut * 2,
                       hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = pad_mask ? hipMemcpyAsync(inf->mask, pad_mask, size_t(P), hipMemcpyDeviceToDevice, s)
                 : hipMemsetAsync(inf->mask, 1, size_t(P), s);
  if (e == hipSuccess) {
    VisPatchParams pp{images, inf->vis->apatch, views};
    e = launch_vis_patch(pp, s);
  }
  if (e == hipSuccess) e = launch_args(args_for(inf->ctx->ws, &kv, noise, actions, 1), s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::launch(g, s);
  if (e == hipSuccess) e = GraphCache<std::pair<int, int>>::mark(g, s);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
  return PI_AE_OK;
}

PI_AE_API void pi_ae_inference_destroy(pi_ae_inference* inf) {
  if (!inf) return;
  {
    DeviceGuard dg(inf->ctx->device);
    inf->release();  // waits for its own launched graphs, then frees
  }
  delete inf;
}

// ====================================================================== guards
PI_AE_API pi_ae_status pi_ae_debug_check_guards(const void* object, int32_t kind, int32_t corrupt,
                                                int32_t* first_bad) {
  if (!object || !first_bad || kind < 0 || kind > 2)
    return fail(PI_AE_EINVAL, "check_guards: object and first_bad non-NULL, kind 0 (expert), 1 (VLM) or 2 (vision)");
  DeviceArena* arena = nullptr;
  int device = 0;
  if (kind == 0) {
    auto* c = static_cast<pi_ae_ctx*>(const_cast<void*>(object));
    arena = &c->arena;
    device = c->device;
  } else if (kind == 1) {
    auto* c = static_cast<pi_ae_vlm*>(const_cast<void*>(object));
    arena = &c->arena;
    device = c->device;
  } else {
    auto* c = static_cast<pi_ae_vision*>(const_cast<void*>(object));
    arena = &c->arena;
    device = c->device;
  }
  DeviceGuard dg(device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) *first_bad = arena->check(corrupt, &e);
  if (e != hipSuccess) return fail(PI_AE_EHIP, std::string("check_guards: ") + hipGetErrorString(e));
  if (*first_bad >= 0)
    return fail(PI_AE_ESTATE, "check_guards: the guard of allocation " + std::to_string(*first_bad) + " changed");
  return PI_AE_OK;
}

PI_AE_API int64_t pi_ae_debug_live_device_bytes(void) { return g_live_device_bytes.load(); }
