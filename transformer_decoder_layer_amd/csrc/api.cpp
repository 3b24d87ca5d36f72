// C-ABI entry points of libtdl: argument checks, handle ownership, the host
// free list of KV blocks, and the per-call launch sequence of the layer.
//
// Launch sequence of one call (the op order of the Qwen2.5-7B single-layer
// page's architecture overview, each step a gfx950 kernel):
//   rmsnorm(x) -> gemm_qkv(+bias) -> rope/q-k norm/kv write -> attention
//   (prefill and/or paged decode) -> gemm_o(+x) -> rmsnorm(h) ->
//   gemm_gate_up(silu gate) -> gemm_down(+h)

#include "../../include/tdl.h"
#include "kernels.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

using namespace tdl;

// The static scratch of layer_decode_paged_noalloc (see scratch_of below).
static __device__ __align__(256) float scratch[(size_t(32) << 20) / sizeof(float)];

namespace {

thread_local std::string g_last_error;

tdl_status fail(tdl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(TDL_E_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                  __LINE__);                                                            \
  } while (0)

bool debug_checks() {
  const char* e = std::getenv("TDL_DEBUG");
  return e && e[0] == '1';
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// ------------------------------------------------------ static scratch
// Device memory of layer_decode_paged_noalloc: the split-K partial slices and
// the decode partitions' partial results of a call live in this array
// instead of the layer's workspace, for callers that cannot allocate.  Each
// GPU the library runs on holds one copy, at its own address, until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: kernels only ever receive the address hipGetSymbolAddress
// returns for the current device (scratch_of).
constexpr size_t kStaticScratchBytes = sizeof(scratch);  // 32 MiB per GPU

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with
// that device current) and kept.
hipError_t scratch_of(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? (float*)p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

// ------------------------------------------------------------------ types

struct tdl_kv_cache {
  tdl_kv_config cfg;
  void* mem = nullptr;
  bool owned = false;
  void* k = nullptr;
  void* v = nullptr;
  float* k_scale = nullptr;
  int32_t* k_zp = nullptr;
  float* v_scale = nullptr;
  int32_t* v_zp = nullptr;
  int8_t* exps = nullptr;  // per-block factor exponents (block_scales)
  std::vector<int32_t> free_list;  // LIFO: back() is handed out next
  std::vector<int32_t> refs;       // holders of each block; 0: on the free list
  // prefix index: key -> (block, last use); the index is one of the block's holders
  struct PrefixEntry {
    int32_t block;
    uint64_t used;
  };
  std::unordered_map<uint64_t, PrefixEntry> prefix;
  std::unordered_map<int32_t, uint64_t> key_of;  // indexed block -> its key
  uint64_t tick = 0;
};

struct tdl_layer {
  tdl_layer_config cfg;
  bool q80 = false;
  bool iq8 = false;  // per-row int8 codes (TDL_I8_ROW)
  bool a8w8 = false;  // int8 weights and activations (TDL_A8W8), scales in w*_rs
  int8_t* aq = nullptr;  // A8W8: int8 codes of a projection's input rows
  float* as = nullptr;   //       and their per-row scales
  // per-row int8: scale and zero point (as floats) of every stored row, in
  // the stored row order (QKV rows concatenated, gate/up interleaved)
  float *wqkv_rs = nullptr, *wqkv_rz = nullptr, *wo_rs = nullptr, *wo_rz = nullptr;
  float *wgu_rs = nullptr, *wgu_rz = nullptr, *wd_rs = nullptr, *wd_rz = nullptr;
  int wexp_packed[4] = {1, 1, 1, 1};  // expanded copies in the packed layout (else row-major)
  int Nqkv = 0;
  // weights (library-owned)
  void* wqkv = nullptr;
  __half* wqkv_s = nullptr;
  float* bqkv = nullptr;
  void* wo = nullptr;
  __half* wo_s = nullptr;
  void* wgu = nullptr;
  __half* wgu_s = nullptr;
  // per weight matrix (QKV, output, gate/up, down): stored in the packed
  // tile layout (bf16/fp16, or per-row int8 codes in the packed code layout,
  // with N % 16 == 0 and K % 64 == 0) or row-major
  int packed[4] = {0, 0, 0, 0};
  // int8 layers that take more than 128 rows: the four matrices expanded to
  // fp16 (bf16 for the down projection), in the packed tile layout where the
  // shape allows, for the compute-bound GEMMs (the decode-sized ones stream
  // the 1-byte codes)
  void* wexp[4] = {nullptr, nullptr, nullptr, nullptr};
  void* wd = nullptr;
  __half* wd_s = nullptr;
  float *ln1 = nullptr, *ln2 = nullptr, *qn = nullptr, *kn = nullptr;
  float2* rope = nullptr;
  // workspace
  void *xn = nullptr, *qkv = nullptr, *q = nullptr, *o = nullptr, *hn = nullptr, *a = nullptr;
  float* h = nullptr;
  float* gemm_ws = nullptr;
  size_t gemm_ws_floats = 0;
  float* dec_part = nullptr;
  size_t dec_part_floats = 0;
  _Float16* stage_k = nullptr;  // prefill staging copies of the new tokens' K / V
  _Float16* stage_v = nullptr;
  int stage_rows = 0;
  void* priv_k = nullptr;  // bf16 pool for calls without a KV cache
  void* priv_v = nullptr;
  int32_t* priv_table = nullptr;  // identity block table of the private pool
  std::vector<void*> allocs;
  // per-stage timing (layer_profile_enable)
  bool prof_on = false;
  struct Mark {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Mark> prof_pending;
  std::vector<hipEvent_t> prof_free;
  double prof_ms[TDL_N_STAGES] = {};
  int64_t prof_n[TDL_N_STAGES] = {};

  ~tdl_layer() {
    for (auto& m : prof_pending) {
      (void)hipEventDestroy(m.a);
      (void)hipEventDestroy(m.b);
    }
    for (auto e : prof_free) (void)hipEventDestroy(e);
    for (void* p : allocs) (void)hipFree(p);
  }
};

namespace {

template <typename T>
tdl_status dalloc(tdl_layer* L, T** out, size_t bytes) {
  void* p = nullptr;
  if (bytes == 0) bytes = 256;
  if (hipMalloc(&p, bytes) != hipSuccess)
    return fail(TDL_E_NOMEM, "hipMalloc of %zu bytes failed", bytes);
  L->allocs.push_back(p);
  *out = (T*)p;
  return TDL_OK;
}

#define TRY(expr)                   \
  do {                              \
    tdl_status s_ = (expr);         \
    if (s_ != TDL_OK) return s_;    \
  } while (0)

tdl_status check_config(const tdl_layer_config* c) {
  if (!c) return fail(TDL_E_INVALID, "config is NULL");
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->intermediate <= 0)
    return fail(TDL_E_INVALID, "non-positive layer dimension");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(TDL_E_INVALID, "n_q_heads (%d) not a multiple of n_kv_heads (%d)", c->n_q_heads,
                c->n_kv_heads);
  const int n_rep = c->n_q_heads / c->n_kv_heads;
  if (!(n_rep == 1 || n_rep == 2 || n_rep == 4 || n_rep == 7 || n_rep == 8))
    return fail(TDL_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4, 7 or 8 (got %d)", n_rep);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(TDL_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->hidden % 64)
    return fail(TDL_E_UNSUPPORTED, "hidden must be a multiple of 64 (got %d)", c->hidden);
  if (c->intermediate % 16)
    return fail(TDL_E_UNSUPPORTED, "intermediate must be a multiple of 16 (got %d)", c->intermediate);
  if (c->weight_dtype != TDL_F32 && c->weight_dtype != TDL_BF16 && c->weight_dtype != TDL_Q8_0 &&
      c->weight_dtype != TDL_I8_ROW && c->weight_dtype != TDL_A8W8)
    return fail(TDL_E_INVALID, "weight_dtype must be TDL_F32, TDL_BF16, TDL_Q8_0, TDL_I8_ROW or TDL_A8W8");
  if ((c->weight_dtype == TDL_Q8_0 || c->weight_dtype == TDL_I8_ROW) &&
      (c->hidden % 32 || c->intermediate % 32 || (c->n_q_heads * c->head_dim) % 32))
    return fail(TDL_E_INVALID, "int8 weights need every input dimension to be a multiple of 32");
  if (c->max_tokens <= 0 || c->max_seqs <= 0 || c->max_position <= 0)
    return fail(TDL_E_INVALID, "max_tokens, max_seqs and max_position must be positive");
  if (std::min(c->max_seqs, c->max_tokens) > kMaxDecodeSeqs || c->max_position > kMaxDecodePosition)
    return fail(TDL_E_UNSUPPORTED, "decode batches above %d sequences or contexts above %d tokens",
                kMaxDecodeSeqs, kMaxDecodePosition);
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f))
    return fail(TDL_E_INVALID, "rms_eps must be >= 0 and rope_theta > 0");
  if (c->rope_fused != 0 && c->rope_fused != 1) return fail(TDL_E_INVALID, "rope_fused must be 0 or 1");
  return TDL_OK;
}

struct GemmShapes {
  int Nqkv, H, Hq_D, I;
};

// Largest split-K workspace over every row count a call may use.
// (per-row int8 layers with expanded copies plan rows > kQ80CodeRows on
// those; Q8_0 layers run on their codes at every row count.)
constexpr int kQ80CodeRows = 128;
void gemm_ws_need(const tdl_layer_config& c, int Nqkv, int wf, bool expanded, size_t* ws) {
  const int H = c.hidden, QD = c.n_q_heads * c.head_dim, I = c.intermediate;
  const int shapes[4][3] = {{Nqkv, H, EPI_BIAS_F32}, {H, QD, EPI_RESID_F32},
                            {2 * I, H, EPI_SILU_GATE}, {H, I, EPI_RESID_BF16}};
  size_t w = 0;
  for (int M = 1; M <= c.max_tokens; ++M) {
    const int f = expanded && M > kQ80CodeRows ? kWDense : wf;
    for (auto& s : shapes) {
      const bool packed = s[0] % 16 == 0 && s[1] % 64 == 0;  // as layer_create packs them
      w = std::max(w, gemm_plan(M, s[0], s[1], f, s[2], f != kWDense && packed).ws_floats);
    }
  }
  *ws = w;
}

// Largest decode partition workspace over every batch size and context bound.
size_t decode_part_need(const tdl_layer_config& c, int max_batch) {
  size_t w = 0;
  const int max_blk = (c.max_position + 15) / 16;
  for (int b = 1; b <= max_batch; ++b)
    for (int fmt : {kKvBf16, kKvU8, kKvU4})
      w = std::max(w, decode_plan(b, c.n_q_heads, c.n_kv_heads, c.head_dim, max_blk * 16, fmt).part_floats_bound);
  return w;
}

KvPool pool_of(const tdl_layer* L, const tdl_kv_cache* kv) {
  KvPool p{};
  if (kv) {
    p.k = kv->k;
    p.v = kv->v;
    p.fmt = kv->cfg.kv_dtype == TDL_U8_ASYM ? kKvU8 : kv->cfg.kv_dtype == TDL_U4_ASYM ? kKvU4 : kKvBf16;
    p.k_scale = kv->k_scale;
    p.k_zp = kv->k_zp;
    p.v_scale = kv->v_scale;
    p.v_zp = kv->v_zp;
    p.exps = kv->exps;
  } else {
    p.k = L->priv_k;
    p.v = L->priv_v;
  }
  return p;
}

// Where one call keeps its partial results: the split-K slices of the GEMMs
// and the decode partitions' (O, m, l).  The layer's own workspace, or the
// library's static scratch (layer_decode_paged_noalloc).  timed: per-stage
// events may be recorded (layer_profile_enable).
struct Scratch {
  float* gemm_ws;
  size_t gemm_floats;
  float* dec_part;
  size_t dec_floats;
  bool timed;
};
Scratch own_scratch(tdl_layer* L) {
  return Scratch{L->gemm_ws, L->gemm_ws_floats, L->dec_part, L->dec_part_floats, true};
}

// Weight format and plan of projection `mat` over M rows: per-row int8
// layers take their expanded copy above kQ80CodeRows rows.
int gemm_format(const tdl_layer* L, int mat, int M) {
  const int wf = L->q80 ? kWQ80 : L->iq8 ? kWIQ8 : kWDense;
  return (wf != kWDense && M > kQ80CodeRows && L->wexp[mat]) ? kWDense : wf;
}

// defer: a split-K plan leaves its fp32 partials in the GEMM workspace for
// the next kernel to sum (*splits_out tells how many; 1 = C was written).
tdl_status run_gemm(tdl_layer* L, const Scratch& sc, hipStream_t st, int mat, int M, int N, int K, const void* A,
                    const void* B, const __half* Bs, const float* Brs, const float* Brz,
                    const void* Bexp, int epi, const float* bias, const void* resid, int ldr, void* C,
                    int ldc, bool defer = false, int* splits_out = nullptr) {
  int wf = L->q80 ? kWQ80 : L->iq8 ? kWIQ8 : kWDense;
  int packed = L->packed[mat];
  // per-row int8 layers: more than kQ80CodeRows rows take the expanded copy
  if (wf != kWDense && M > kQ80CodeRows && Bexp) {
    wf = kWDense;
    B = Bexp;
    Bs = nullptr;
    packed = L->wexp_packed[mat];
  }
  if (wf == kWIQ8 && M > kQ80CodeRows)
    return fail(TDL_E_UNSUPPORTED, "per-row int8 weights without an expanded copy at M=%d", M);
  const GemmPlan pl = gemm_plan(M, N, K, wf, epi, wf != kWDense && packed);
  if (splits_out) *splits_out = defer ? pl.splits : 1;
  if (pl.ws_floats > sc.gemm_floats)
    return fail(TDL_E_CAPACITY, "GEMM workspace too small for M=%d N=%d K=%d", M, N, K);
  GemmArgs a{};
  a.A = A;
  a.lda = K;
  a.B = B;
  a.ldb = K;
  a.B_scale = Bs;
  a.B_rscale = wf == kWIQ8 ? Brs : nullptr;
  a.B_rzp = wf == kWIQ8 ? Brz : nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.bias = bias;
  a.resid = resid;
  a.ldr = ldr;
  a.C = C;
  a.ldc = ldc;
  a.ws = sc.gemm_ws;
  a.b_packed = packed;
  HIP_TRY(gemm_launch(pl, a, wf, epi, st, !defer));
  return TDL_OK;
}

// Per-stage timing: a StageTimer records an event pair around one stage's
// kernels on the call's stream while profiling is on.
hipEvent_t take_event(tdl_layer* L) {
  if (!L->prof_free.empty()) {
    hipEvent_t e = L->prof_free.back();
    L->prof_free.pop_back();
    return e;
  }
  // timing-only events: without the system-scope fence a recorded event
  // does not write back and invalidate the caches, which would start every
  // following stage cold and inflate its time
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}
int prof_begin(tdl_layer* L, int stage, hipStream_t st) {
  if (!L->prof_on) return -1;
  tdl_layer::Mark m{stage, take_event(L), take_event(L)};
  if (!m.a || !m.b) return -1;
  (void)hipEventRecord(m.a, st);
  L->prof_pending.push_back(m);
  return (int)L->prof_pending.size() - 1;
}
struct StageTimer {
  tdl_layer* L;
  hipStream_t st;
  int mark;
  StageTimer(tdl_layer* l, int stage, hipStream_t s, bool timed = true)
      : L(l), st(s), mark(timed ? prof_begin(l, stage, s) : -1) {}
  ~StageTimer() {
    if (mark >= 0) (void)hipEventRecord(L->prof_pending[mark].b, st);
  }
};

// A8W8 projection `mat` (0 QKV, 1 output, 2 gate/up, 3 down) over M rows:
// the input rows A (fp16, or bf16 for the down projection) to int8 with a
// scale per row, then the int8 GEMM, dequantised with both scales and
// finished by the projection's epilogue in the GEMM kernel (QKV + bias ->
// qkv; + x -> h; SiLU(gate) * up -> a; + h -> y).
tdl_status a8w8_project(tdl_layer* L, hipStream_t st, int mat, int M, int N, int K, const void* A,
                        const void* resid, void* out) {
  HIP_TRY(quant_rows_i8(A, mat == 3, M, K, L->aq, L->as, st));
  const void* B = mat == 0 ? L->wqkv : mat == 1 ? L->wo : mat == 2 ? L->wgu : L->wd;
  const float* bs = mat == 0 ? L->wqkv_rs : mat == 1 ? L->wo_rs : mat == 2 ? L->wgu_rs : L->wd_rs;
  A8Epi e{};
  e.epi = mat == 0 ? kA8Bias : mat == 1 ? kA8ResidF32 : mat == 2 ? kA8SiluGate : kA8ResidBf16;
  e.bias = mat == 0 ? L->bqkv : nullptr;
  e.resid = resid;
  e.ldr = L->cfg.hidden;
  e.out = out;
  e.ldo = mat == 2 ? N / 2 : N;
  HIP_TRY(a8w8_gemm_epi(L->aq, B, L->as, bs, nullptr, e, M, N, K, st));
  return TDL_OK;
}

// The whole layer over `rows` rows.  Sequences 0..n_prefill-1 of `seq` use the
// prefill attention kernel, decode sequences dec_first .. dec_first+n_dec-1
// the paged decode kernel.
constexpr int kFusedNormMaxH = 8192;  // hidden sizes the fused split-sum RMSNorm takes

tdl_status run_layer(tdl_layer* L, const Scratch& sc, hipStream_t st, const void* x, void* y,
                     int rows, SeqInfo seq, KvPool pool, int n_prefill, int max_q_len, int dec_first,
                     int n_dec, int max_ctx_len) {
  const tdl_layer_config& c = L->cfg;
  const int H = c.hidden, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads, I = c.intermediate;
  DecodePlan dp{};
  if (n_dec) {
    dp = decode_plan(n_dec, Hq, Hkv, D, max_ctx_len, pool.fmt);
    if (dp.part_floats > sc.dec_floats)
      return fail(TDL_E_CAPACITY, "decode workspace too small (batch %d, max_ctx_len %d)", n_dec,
                  max_ctx_len);
  }
  {
    StageTimer t(L, TDL_STAGE_RMSNORM1, st, sc.timed);
    HIP_TRY(rmsnorm_bf16in(x, L->ln1, L->xn, rows, H, c.rms_eps, st));
  }
  // a split QKV projection is summed (with its bias) by the RoPE kernel, and
  // a split output projection (with the residual) by RMSNorm-2: two fewer
  // launches and no second round trip of the sums
  int qkv_splits = 1;
  PrefillStage stage{L->stage_k, L->stage_v, L->stage_rows, std::min(n_prefill, kStagedSeqs)};
  {
    StageTimer t(L, TDL_STAGE_QKV, st, sc.timed);
    if (L->a8w8)
      TRY(a8w8_project(L, st, 0, rows, L->Nqkv, H, L->xn, nullptr, L->qkv));
    else
      TRY(run_gemm(L, sc, st, 0, rows, L->Nqkv, H, L->xn, L->wqkv, L->wqkv_s, L->wqkv_rs, L->wqkv_rz, L->wexp[0], EPI_BIAS_F32, L->bqkv, nullptr,
                   0, L->qkv, L->Nqkv, true, &qkv_splits));
  }
  // rope_fused: the prefill rows' queries go from the (whole, unsplit) QKV
  // projection, bias included, straight into the prefill attention kernel,
  // which applies the Q-norm and RoPE as it loads them.  A projection split
  // along K keeps the RoPE kernel's q: summing the slices in the attention
  // kernel's prologue cost it more than the RoPE kernel saved (512 tokens:
  // attention +9 us, RoPE -7 us).
  const bool q_fused = c.rope_fused && n_prefill > 0 && qkv_splits == 1;
  PrefillQ qsrc{};
  if (q_fused)
    qsrc = PrefillQ{(const float*)L->qkv, L->Nqkv, nullptr, c.qk_norm ? L->qn : nullptr, c.rms_eps, L->rope};
  {
    StageTimer t(L, TDL_STAGE_ROPE_KV, st, sc.timed);
    HIP_TRY(rope_kv_write(qkv_splits > 1 ? (const void*)sc.gemm_ws : (const void*)L->qkv, rows, Hq, Hkv,
                          D, L->rope, c.qk_norm ? L->qn : nullptr, c.qk_norm ? L->kn : nullptr,
                          c.rms_eps, L->q, seq, pool, stage, st, qkv_splits,
                          qkv_splits > 1 ? L->bqkv : nullptr, q_fused ? n_prefill : 0));
  }
  if (n_prefill) {
    StageTimer t(L, TDL_STAGE_ATTN_PREFILL, st, sc.timed);
    HIP_TRY(attn_prefill(L->q, qsrc, pool, seq, stage, n_prefill, max_q_len, Hq, Hkv, D, L->o, st));
  }
  if (n_dec) {
    StageTimer t(L, TDL_STAGE_ATTN_DECODE, st, sc.timed);
    HIP_TRY(attn_decode(dp, L->q, pool, seq, dec_first, n_dec, Hq, Hkv, D, L->o, sc.dec_part, st));
  }
  if (L->a8w8) {
    {
      StageTimer t(L, TDL_STAGE_O_PROJ, st, sc.timed);
      TRY(a8w8_project(L, st, 1, rows, H, Hq * D, L->o, x, L->h));
    }
    {
      StageTimer t(L, TDL_STAGE_RMSNORM2, st, sc.timed);
      HIP_TRY(rmsnorm_f32in(L->h, L->ln2, L->hn, rows, H, c.rms_eps, st));
    }
    {
      StageTimer t(L, TDL_STAGE_GATE_UP, st, sc.timed);
      TRY(a8w8_project(L, st, 2, rows, 2 * I, H, L->hn, nullptr, L->a));
    }
    {
      StageTimer t(L, TDL_STAGE_DOWN, st, sc.timed);
      TRY(a8w8_project(L, st, 3, rows, H, I, L->a, L->h, y));
    }
    return TDL_OK;
  }
  int o_splits = 1;
  {
    StageTimer t(L, TDL_STAGE_O_PROJ, st, sc.timed);
    TRY(run_gemm(L, sc, st, 1, rows, H, Hq * D, L->o, L->wo, L->wo_s, L->wo_rs, L->wo_rz, L->wexp[1], EPI_RESID_F32, nullptr, x, H, L->h,
                 H, H <= kFusedNormMaxH, &o_splits));
  }
  {
    StageTimer t(L, TDL_STAGE_RMSNORM2, st, sc.timed);
    if (o_splits > 1)
      HIP_TRY(rmsnorm_splits_resid(sc.gemm_ws, o_splits, x, L->h, L->ln2, L->hn, rows, H, c.rms_eps, st));
    else
      HIP_TRY(rmsnorm_f32in(L->h, L->ln2, L->hn, rows, H, c.rms_eps, st));
  }
  {
    StageTimer t(L, TDL_STAGE_GATE_UP, st, sc.timed);
    TRY(run_gemm(L, sc, st, 2, rows, 2 * I, H, L->hn, L->wgu, L->wgu_s, L->wgu_rs, L->wgu_rz, L->wexp[2], EPI_SILU_GATE, nullptr, nullptr, 0,
                 L->a, I));
  }
  {
    StageTimer t(L, TDL_STAGE_DOWN, st, sc.timed);
    TRY(run_gemm(L, sc, st, 3, rows, H, I, L->a, L->wd, L->wd_s, L->wd_rs, L->wd_rz, L->wexp[3], EPI_RESID_BF16, nullptr, L->h, H, y, H));
  }
  return TDL_OK;
}

tdl_status check_kv_matches(const tdl_layer* L, const tdl_kv_cache* kv) {
  if (!kv) return TDL_OK;
  if (kv->cfg.n_kv_heads != L->cfg.n_kv_heads || kv->cfg.head_dim != L->cfg.head_dim)
    return fail(TDL_E_INVALID, "KV cache heads/head_dim do not match the layer");
  return TDL_OK;
}

// TDL_DEBUG=1: copy device tables back and check every entry a call will read.
tdl_status debug_check_tables(const int32_t* ctx_dev, const int32_t* qlen_dev, int n, int extra,
                              const int32_t* tables_dev, int max_blocks, int n_blocks,
                              int max_ctx_len, hipStream_t st) {
  std::vector<int32_t> ctx(n), qlen(n, extra), tab((size_t)n * max_blocks);
  HIP_TRY(hipStreamSynchronize(st));
  HIP_TRY(hipMemcpy(ctx.data(), ctx_dev, n * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (qlen_dev) HIP_TRY(hipMemcpy(qlen.data(), qlen_dev, n * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(tab.data(), tables_dev, tab.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
  for (int i = 0; i < n; ++i) {
    const int total = ctx[i] + qlen[i];
    if (ctx[i] < 0 || total > max_ctx_len)
      return fail(TDL_E_INVALID, "sequence %d: ctx_len %d + %d exceeds max_ctx_len %d", i, ctx[i],
                  qlen[i], max_ctx_len);
    for (int b = 0; b < (total + 15) / 16; ++b) {
      const int blk = tab[(size_t)i * max_blocks + b];
      if (blk < 0 || blk >= n_blocks)
        return fail(TDL_E_INVALID, "sequence %d: block table entry %d = %d out of range", i, b, blk);
    }
  }
  return TDL_OK;
}

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

}  // namespace

// ================================================================ layer

extern "C" tdl_status layer_create(const tdl_layer_config* cfg, const tdl_layer_weights* w,
                                   tdl_stream stream, tdl_layer** out) {
  if (!out) return fail(TDL_E_INVALID, "out is NULL");
  *out = nullptr;
  TRY(check_config(cfg));
  if (!w) return fail(TDL_E_INVALID, "weights are NULL");
  const tdl_layer_config& c = *cfg;
  const bool q80 = c.weight_dtype == TDL_Q8_0;
  const bool iq8 = c.weight_dtype == TDL_I8_ROW;
  const bool a8w8 = c.weight_dtype == TDL_A8W8;
  const bool codes = q80 || iq8 || a8w8;  // 1-byte codes stored as given
  if (!w->ln1 || !w->wq || !w->wk || !w->wv || !w->wo || !w->ln2 || !w->wg || !w->wu || !w->wd)
    return fail(TDL_E_INVALID, "a required weight pointer is NULL");
  if (c.qkv_bias && (!w->bq || !w->bk || !w->bv))
    return fail(TDL_E_INVALID, "qkv_bias set but a bias pointer is NULL");
  if (c.qk_norm && (!w->q_norm || !w->k_norm))
    return fail(TDL_E_INVALID, "qk_norm set but q_norm/k_norm is NULL");
  if (q80 && (!w->wq_scale || !w->wk_scale || !w->wv_scale || !w->wo_scale || !w->wg_scale ||
              !w->wu_scale || !w->wd_scale))
    return fail(TDL_E_INVALID, "Q8_0 weights need every *_scale pointer");
  if (iq8 && (!w->wq_scale || !w->wk_scale || !w->wv_scale || !w->wo_scale || !w->wg_scale ||
              !w->wu_scale || !w->wd_scale || !w->wq_zp || !w->wk_zp || !w->wv_zp || !w->wo_zp ||
              !w->wg_zp || !w->wu_zp || !w->wd_zp))
    return fail(TDL_E_INVALID, "per-row int8 weights need every *_scale and *_zp pointer");
  if (a8w8 && (!w->wq_scale || !w->wk_scale || !w->wv_scale || !w->wo_scale || !w->wg_scale ||
               !w->wu_scale || !w->wd_scale))
    return fail(TDL_E_INVALID, "A8W8 weights need every *_scale pointer");

  hipStream_t st = (hipStream_t)stream;
  {
    // set-up of the static scratch on this device (layer_decode_paged_noalloc)
    float* sp = nullptr;
    const hipError_t e = scratch_of(&sp);
    if (e != hipSuccess) return fail(TDL_E_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
  }
  tdl_layer* L = new tdl_layer();
  L->cfg = c;
  L->q80 = q80;
  L->iq8 = iq8;
  L->a8w8 = a8w8;
  const int H = c.hidden, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads, I = c.intermediate;
  const int QD = Hq * D, KD = Hkv * D;
  L->Nqkv = QD + 2 * KD;
  const int T = c.max_tokens;
  auto bail = [&](tdl_status s) {
    delete L;
    return s;
  };
#define CTRY(expr)                        \
  do {                                    \
    tdl_status s2_ = (expr);              \
    if (s2_ != TDL_OK) return bail(s2_);  \
  } while (0)
#define CHIP(expr)                                                                            \
  do {                                                                                        \
    hipError_t e2_ = (expr);                                                                  \
    if (e2_ != hipSuccess)                                                                    \
      return bail(fail(TDL_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e2_)));          \
  } while (0)

  // ---- weights: bf16 copies (f32 rounded to nearest even), or Q8_0 codes
  const size_t wel = codes ? 1 : 2;  // bytes per stored weight element
  CTRY(dalloc(L, &L->wqkv, (size_t)L->Nqkv * H * wel));
  CTRY(dalloc(L, &L->wo, (size_t)H * QD * wel));
  CTRY(dalloc(L, &L->wgu, (size_t)2 * I * H * wel));
  CTRY(dalloc(L, &L->wd, (size_t)H * I * wel));
  // fp16 copies for the projections whose activation input is bounded (QKV,
  // output, gate/up); bf16 for the down projection.  Saturated fp16 values
  // are counted and refused below.
  int* n_sat = nullptr;
  CTRY(dalloc(L, &n_sat, 4));
  CHIP(hipMemsetAsync(n_sat, 0, 4, st));
  auto put = [&](const void* src, void* dst, int64_t n, int to_f16) -> tdl_status {
    const hipError_t e = codes ? hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, st)
                             : convert_weights(src, c.weight_dtype == TDL_F32, dst, to_f16, n,
                                               n_sat, st);
    if (e != hipSuccess) return fail(TDL_E_HIP, "weight copy failed: %s", hipGetErrorString(e));
    return TDL_OK;
  };
  char* qkv = (char*)L->wqkv;
  CTRY(put(w->wq, qkv, (int64_t)QD * H, 1));
  CTRY(put(w->wk, qkv + (size_t)QD * H * wel, (int64_t)KD * H, 1));
  CTRY(put(w->wv, qkv + (size_t)(QD + KD) * H * wel, (int64_t)KD * H, 1));
  CTRY(put(w->wo, L->wo, (int64_t)H * QD, 1));
  CTRY(put(w->wd, L->wd, (int64_t)H * I, 0));
  {
    // gate/up: convert to the stored type, then interleave 16-row groups
    void* g16 = nullptr;
    void* u16 = nullptr;
    CTRY(dalloc(L, &g16, (size_t)I * H * wel));
    CTRY(dalloc(L, &u16, (size_t)I * H * wel));
    CTRY(put(w->wg, g16, (int64_t)I * H, 1));
    CTRY(put(w->wu, u16, (int64_t)I * H, 1));
    CHIP(interleave_gate_up(g16, u16, (int)(H * wel), I, L->wgu, st));
    CHIP(hipStreamSynchronize(st));
    for (void* p : {g16, u16}) {
      L->allocs.erase(std::find(L->allocs.begin(), L->allocs.end(), p));
      (void)hipFree(p);
    }
  }
  if (!codes) {
    // repack every matrix the tiled readers can take (one temporary the size
    // of the largest)
    const int shapes[4][2] = {{L->Nqkv, H}, {H, QD}, {2 * I, H}, {H, I}};
    void* mats[4] = {L->wqkv, L->wo, L->wgu, L->wd};
    size_t most = 0;
    for (auto& sh : shapes) most = std::max(most, (size_t)sh[0] * sh[1] * 2);
    void* tmp = nullptr;
    CTRY(dalloc(L, &tmp, most));
    for (int i = 0; i < 4; ++i) {
      if (shapes[i][0] % 16 != 0 || shapes[i][1] % 64 != 0) continue;
      CHIP(pack_weights(mats[i], tmp, shapes[i][0], shapes[i][1], st));
      CHIP(hipMemcpyAsync(mats[i], tmp, (size_t)shapes[i][0] * shapes[i][1] * 2,
                          hipMemcpyDeviceToDevice, st));
      L->packed[i] = 1;
    }
    CHIP(hipStreamSynchronize(st));
    L->allocs.erase(std::find(L->allocs.begin(), L->allocs.end(), tmp));
    (void)hipFree(tmp);
  }
  if (q80) {
    CTRY(dalloc(L, &L->wqkv_s, (size_t)L->Nqkv * (H / 32) * 2));
    CTRY(dalloc(L, &L->wo_s, (size_t)H * (QD / 32) * 2));
    CTRY(dalloc(L, &L->wgu_s, (size_t)2 * I * (H / 32) * 2));
    CTRY(dalloc(L, &L->wd_s, (size_t)H * (I / 32) * 2));
    char* s = (char*)L->wqkv_s;
    const size_t rs = (size_t)(H / 32) * 2;
    CHIP(hipMemcpyAsync(s, w->wq_scale, QD * rs, hipMemcpyDeviceToDevice, st));
    CHIP(hipMemcpyAsync(s + QD * rs, w->wk_scale, KD * rs, hipMemcpyDeviceToDevice, st));
    CHIP(hipMemcpyAsync(s + (QD + KD) * rs, w->wv_scale, KD * rs, hipMemcpyDeviceToDevice, st));
    CHIP(hipMemcpyAsync(L->wo_s, w->wo_scale, (size_t)H * (QD / 32) * 2, hipMemcpyDeviceToDevice, st));
    CHIP(hipMemcpyAsync(L->wd_s, w->wd_scale, (size_t)H * (I / 32) * 2, hipMemcpyDeviceToDevice, st));
    CHIP(interleave_gate_up(w->wg_scale, w->wu_scale, (int)rs, I, L->wgu_s, st));
    CHIP(hipStreamSynchronize(st));
  }
  if (a8w8) {
    // per-row scales (float32, copied) in the stored row order; gate/up rows
    // interleaved like the codes (which stay row-major: the int8 GEMM reads
    // them so)
    auto rows_f32 = [&](float** dst, int n) { return dalloc(L, dst, (size_t)n * 4); };
    CTRY(rows_f32(&L->wqkv_rs, L->Nqkv));
    CTRY(rows_f32(&L->wo_rs, H));
    CTRY(rows_f32(&L->wgu_rs, 2 * I));
    CTRY(rows_f32(&L->wd_rs, H));
    CHIP(copy_f32((const float*)w->wq_scale, L->wqkv_rs, QD, st));
    CHIP(copy_f32((const float*)w->wk_scale, L->wqkv_rs + QD, KD, st));
    CHIP(copy_f32((const float*)w->wv_scale, L->wqkv_rs + QD + KD, KD, st));
    CHIP(copy_f32((const float*)w->wo_scale, L->wo_rs, H, st));
    CHIP(copy_f32((const float*)w->wd_scale, L->wd_rs, H, st));
    CHIP(interleave_gate_up(w->wg_scale, w->wu_scale, 4, I, L->wgu_rs, st));
    CHIP(hipStreamSynchronize(st));
  }
  if (iq8) {
    // per-row scales (float32, copied) and zero points (int8 -> float), in
    // the stored row order; gate/up rows interleaved like the codes
    auto rows_f32 = [&](float** dst, int n) { return dalloc(L, dst, (size_t)n * 4); };
    CTRY(rows_f32(&L->wqkv_rs, L->Nqkv));
    CTRY(rows_f32(&L->wqkv_rz, L->Nqkv));
    CTRY(rows_f32(&L->wo_rs, H));
    CTRY(rows_f32(&L->wo_rz, H));
    CTRY(rows_f32(&L->wgu_rs, 2 * I));
    CTRY(rows_f32(&L->wgu_rz, 2 * I));
    CTRY(rows_f32(&L->wd_rs, H));
    CTRY(rows_f32(&L->wd_rz, H));
    CHIP(copy_f32((const float*)w->wq_scale, L->wqkv_rs, QD, st));
    CHIP(copy_f32((const float*)w->wk_scale, L->wqkv_rs + QD, KD, st));
    CHIP(copy_f32((const float*)w->wv_scale, L->wqkv_rs + QD + KD, KD, st));
    CHIP(i8_to_f32(w->wq_zp, L->wqkv_rz, QD, st));
    CHIP(i8_to_f32(w->wk_zp, L->wqkv_rz + QD, KD, st));
    CHIP(i8_to_f32(w->wv_zp, L->wqkv_rz + QD + KD, KD, st));
    CHIP(copy_f32((const float*)w->wo_scale, L->wo_rs, H, st));
    CHIP(i8_to_f32(w->wo_zp, L->wo_rz, H, st));
    CHIP(copy_f32((const float*)w->wd_scale, L->wd_rs, H, st));
    CHIP(i8_to_f32(w->wd_zp, L->wd_rz, H, st));
    float* gz = nullptr;
    float* uz = nullptr;
    CTRY(rows_f32(&gz, I));
    CTRY(rows_f32(&uz, I));
    CHIP(i8_to_f32(w->wg_zp, gz, I, st));
    CHIP(i8_to_f32(w->wu_zp, uz, I, st));
    CHIP(interleave_gate_up(w->wg_scale, w->wu_scale, 4, I, L->wgu_rs, st));
    CHIP(interleave_gate_up(gz, uz, 4, I, L->wgu_rz, st));
    CHIP(hipStreamSynchronize(st));
    for (void* p : {(void*)gz, (void*)uz}) {
      L->allocs.erase(std::find(L->allocs.begin(), L->allocs.end(), p));
      (void)hipFree(p);
    }
    if (c.max_tokens > kQ80CodeRows) {
      // expanded copies for the compute-bound GEMMs: packed where the shape
      // allows, row-major otherwise (the large-M kernels have no int8 path)
      const int shapes[4][2] = {{L->Nqkv, H}, {H, QD}, {2 * I, H}, {H, I}};
      const void* cm[4] = {L->wqkv, L->wo, L->wgu, L->wd};
      const float* rs[4] = {L->wqkv_rs, L->wo_rs, L->wgu_rs, L->wd_rs};
      const float* rz[4] = {L->wqkv_rz, L->wo_rz, L->wgu_rz, L->wd_rz};
      size_t most = 0;
      for (auto& sh : shapes) most = std::max(most, (size_t)sh[0] * sh[1] * 2);
      void* tmp = nullptr;
      CTRY(dalloc(L, &tmp, most));
      for (int i = 0; i < 4; ++i) {
        const bool pk = shapes[i][0] % 16 == 0 && shapes[i][1] % 64 == 0;
        CTRY(dalloc(L, &L->wexp[i], (size_t)shapes[i][0] * shapes[i][1] * 2));
        CHIP(expand_iq8(cm[i], rs[i], rz[i], shapes[i][0], shapes[i][1], pk ? tmp : L->wexp[i],
                        i != 3, st));
        if (pk) CHIP(pack_weights(tmp, L->wexp[i], shapes[i][0], shapes[i][1], st));
        L->wexp_packed[i] = pk;
      }
      CHIP(hipStreamSynchronize(st));
      L->allocs.erase(std::find(L->allocs.begin(), L->allocs.end(), tmp));
      (void)hipFree(tmp);
    }
  }
  if (q80 || iq8) {
    // the codes themselves in the packed code layout where the shape allows
    // (the stream kernel: one contiguous 1 KB read per wave and stage; the
    // large-M Q8_0 kernel: one direct 1 KB copy per 16 rows and 64 k); after
    // any expansion above, which reads them row-major
    const int shapes[4][2] = {{L->Nqkv, H}, {H, QD}, {2 * I, H}, {H, I}};
    void* mats[4] = {L->wqkv, L->wo, L->wgu, L->wd};
    size_t most = 0;
    for (auto& sh : shapes) most = std::max(most, (size_t)sh[0] * sh[1]);
    void* tmp = nullptr;
    CTRY(dalloc(L, &tmp, most));
    for (int i = 0; i < 4; ++i) {
      if (shapes[i][0] % 16 != 0 || shapes[i][1] % 64 != 0) continue;
      CHIP(pack_codes(mats[i], tmp, shapes[i][0], shapes[i][1], st));
      CHIP(hipMemcpyAsync(mats[i], tmp, (size_t)shapes[i][0] * shapes[i][1], hipMemcpyDeviceToDevice, st));
      L->packed[i] = 1;
    }
    CHIP(hipStreamSynchronize(st));
    L->allocs.erase(std::find(L->allocs.begin(), L->allocs.end(), tmp));
    (void)hipFree(tmp);
  }
  if (c.qkv_bias) {
    CTRY(dalloc(L, &L->bqkv, (size_t)L->Nqkv * 4));
    CHIP(copy_f32((const float*)w->bq, L->bqkv, QD, st));
    CHIP(copy_f32((const float*)w->bk, L->bqkv + QD, KD, st));
    CHIP(copy_f32((const float*)w->bv, L->bqkv + QD + KD, KD, st));
  }
  CTRY(dalloc(L, &L->ln1, (size_t)H * 4));
  CTRY(dalloc(L, &L->ln2, (size_t)H * 4));
  CHIP(copy_f32((const float*)w->ln1, L->ln1, H, st));
  CHIP(copy_f32((const float*)w->ln2, L->ln2, H, st));
  if (c.qk_norm) {
    CTRY(dalloc(L, &L->qn, (size_t)D * 4));
    CTRY(dalloc(L, &L->kn, (size_t)D * 4));
    CHIP(copy_f32((const float*)w->q_norm, L->qn, D, st));
    CHIP(copy_f32((const float*)w->k_norm, L->kn, D, st));
  }
  CTRY(dalloc(L, &L->rope, (size_t)c.max_position * (D / 2) * sizeof(float2)));
  CHIP(rope_table_build(L->rope, c.max_position, D, (double)c.rope_theta, st));

  // ---- workspace
  CTRY(dalloc(L, &L->xn, (size_t)T * H * 2));
  CTRY(dalloc(L, &L->qkv, (size_t)T * L->Nqkv * 4));
  CTRY(dalloc(L, &L->q, (size_t)T * QD * 4));
  CTRY(dalloc(L, &L->o, (size_t)T * QD * 2));
  CTRY(dalloc(L, &L->h, (size_t)T * H * 4));
  CTRY(dalloc(L, &L->hn, (size_t)T * H * 2));
  CTRY(dalloc(L, &L->a, (size_t)T * I * 2));
  gemm_ws_need(c, L->Nqkv, q80 ? kWQ80 : iq8 ? kWIQ8 : kWDense, L->wexp[0] != nullptr,
               &L->gemm_ws_floats);
  if (a8w8) {
    // the int8 codes and scales of the widest projection input
    CTRY(dalloc(L, &L->aq, (size_t)T * std::max({H, QD, I})));
    CTRY(dalloc(L, &L->as, (size_t)T * 4));
  }
  CTRY(dalloc(L, &L->gemm_ws, L->gemm_ws_floats * 4));
  const int max_dec = std::min(c.max_seqs, c.max_tokens);
  L->dec_part_floats = decode_part_need(c, max_dec);
  CTRY(dalloc(L, &L->dec_part, L->dec_part_floats * 4));
  // prefill staging: K and V of the new tokens as fp16, zeroed once so that
  // rows no call has written hold finite values
  L->stage_rows = prefill_stage_rows(T);
  {
    const size_t sb = (size_t)KD * L->stage_rows * sizeof(_Float16);
    CTRY(dalloc(L, &L->stage_k, sb));
    CTRY(dalloc(L, &L->stage_v, sb));
    CHIP(hipMemsetAsync(L->stage_k, 0, sb, st));
    CHIP(hipMemsetAsync(L->stage_v, 0, sb, st));
  }
  const size_t priv_blocks = (size_t)(T + 15) / 16;
  CTRY(dalloc(L, &L->priv_k, priv_blocks * KD * 16 * 2));
  CTRY(dalloc(L, &L->priv_v, priv_blocks * KD * 16 * 2));
  CTRY(dalloc(L, &L->priv_table, priv_blocks * sizeof(int32_t)));
  {
    std::vector<int32_t> ident(priv_blocks);
    for (size_t b = 0; b < priv_blocks; ++b) ident[b] = (int32_t)b;
    CHIP(hipMemcpy(L->priv_table, ident.data(), priv_blocks * sizeof(int32_t), hipMemcpyHostToDevice));
  }
  CHIP(hipStreamSynchronize(st));
  int sat = 0;
  CHIP(hipMemcpy(&sat, n_sat, 4, hipMemcpyDeviceToHost));
  if (sat)
    return bail(fail(TDL_E_UNSUPPORTED, "%d weights exceed the fp16 range (|w| > 65504)", sat));
  *out = L;
  return TDL_OK;
#undef CTRY
#undef CHIP
}

extern "C" tdl_status layer_destroy(tdl_layer* layer) {
  delete layer;
  return TDL_OK;
}

extern "C" tdl_status layer_prefill(tdl_layer* L, tdl_stream stream, const void* x, void* y,
                                    int32_t n_tokens, int32_t start_pos, tdl_kv_cache* kv,
                                    const int32_t* block_table) {
  if (!L) return fail(TDL_E_INVALID, "layer is NULL");
  if (!x || !y) return fail(TDL_E_INVALID, "x or y is NULL");
  if (x == y) return fail(TDL_E_INVALID, "y must not alias x");
  if (((uintptr_t)x | (uintptr_t)y) & 15) return fail(TDL_E_INVALID, "x and y must be 16-byte aligned");
  if (n_tokens < 1 || n_tokens > L->cfg.max_tokens)
    return fail(n_tokens < 1 ? TDL_E_INVALID : TDL_E_CAPACITY,
                "n_tokens %d outside [1, max_tokens=%d]", n_tokens, L->cfg.max_tokens);
  if (start_pos < 0) return fail(TDL_E_INVALID, "start_pos < 0");
  if ((int64_t)start_pos + n_tokens > L->cfg.max_position)
    return fail(TDL_E_CAPACITY, "positions up to %d exceed max_position %d",
                start_pos + n_tokens - 1, L->cfg.max_position);
  if (!kv && start_pos != 0) return fail(TDL_E_INVALID, "start_pos > 0 needs a KV cache");
  if (kv && !block_table) return fail(TDL_E_INVALID, "a KV cache needs a block table");
  TRY(check_kv_matches(L, kv));
  const int total = start_pos + n_tokens;
  if (kv && total > kv->cfg.n_blocks * 16)
    return fail(TDL_E_CAPACITY, "sequence longer than the cache pool");
  hipStream_t st = (hipStream_t)stream;
  if (kv && debug_checks()) {
    int32_t ctx_h = start_pos;
    (void)ctx_h;
    std::vector<int32_t> tab((total + 15) / 16);
    HIP_TRY(hipStreamSynchronize(st));
    HIP_TRY(hipMemcpy(tab.data(), block_table, tab.size() * 4, hipMemcpyDeviceToHost));
    for (size_t b = 0; b < tab.size(); ++b)
      if (tab[b] < 0 || tab[b] >= kv->cfg.n_blocks)
        return fail(TDL_E_INVALID, "block table entry %zu = %d out of range", b, tab[b]);
  }
  SeqInfo seq{};
  seq.n_seqs = 1;
  seq.q_len0 = n_tokens;
  seq.ctx0 = start_pos;
  seq.tables = kv ? block_table : L->priv_table;
  seq.max_blocks = 0;
  return run_layer(L, own_scratch(L), st, x, y, n_tokens, seq, pool_of(L, kv), 1, n_tokens, 0, 0, 0);
}

// Host-side checks of a decode step (nothing is enqueued).
tdl_status check_decode(const tdl_layer* L, const void* x, const void* y, int32_t batch,
                        const int32_t* ctx_lens, const int32_t* block_tables, int32_t max_blocks,
                        int32_t max_ctx_len, const tdl_kv_cache* kv) {
  if (!L) return fail(TDL_E_INVALID, "layer is NULL");
  if (!x || !y || !ctx_lens || !block_tables || !kv)
    return fail(TDL_E_INVALID, "x, y, ctx_lens, block_tables and kv are required");
  if (x == y) return fail(TDL_E_INVALID, "y must not alias x");
  if (((uintptr_t)x | (uintptr_t)y) & 15) return fail(TDL_E_INVALID, "x and y must be 16-byte aligned");
  if (batch < 1) return fail(TDL_E_INVALID, "batch < 1");
  if (batch > L->cfg.max_seqs || batch > L->cfg.max_tokens)
    return fail(TDL_E_CAPACITY, "batch %d exceeds max_seqs/max_tokens", batch);
  if (max_blocks < 1) return fail(TDL_E_INVALID, "max_blocks < 1");
  if (max_ctx_len < 1 || max_ctx_len > max_blocks * 16)
    return fail(TDL_E_INVALID, "max_ctx_len %d outside [1, max_blocks*16]", max_ctx_len);
  if (max_ctx_len > L->cfg.max_position)
    return fail(TDL_E_CAPACITY, "max_ctx_len %d exceeds max_position %d", max_ctx_len,
                L->cfg.max_position);
  return check_kv_matches(L, kv);
}

tdl_status enqueue_decode(tdl_layer* L, const Scratch& sc, hipStream_t st, const void* x, void* y,
                          int32_t batch, const int32_t* ctx_lens, const int32_t* block_tables,
                          int32_t max_blocks, int32_t max_ctx_len, tdl_kv_cache* kv) {
  if (sc.timed && debug_checks())
    TRY(debug_check_tables(ctx_lens, nullptr, batch, 1, block_tables, max_blocks, kv->cfg.n_blocks,
                           max_ctx_len, st));
  SeqInfo seq{};
  seq.ctx_len = ctx_lens;
  seq.n_seqs = batch;
  seq.tables = block_tables;
  seq.max_blocks = max_blocks;
  seq.rows_are_seqs = 1;
  return run_layer(L, sc, st, x, y, batch, seq, pool_of(L, kv), 0, 0, 0, batch, max_ctx_len);
}

extern "C" tdl_status layer_decode_paged(tdl_layer* L, tdl_stream stream, const void* x, void* y,
                                         int32_t batch, const int32_t* ctx_lens,
                                         const int32_t* block_tables, int32_t max_blocks,
                                         int32_t max_ctx_len, tdl_kv_cache* kv) {
  TRY(check_decode(L, x, y, batch, ctx_lens, block_tables, max_blocks, max_ctx_len, kv));
  return enqueue_decode(L, own_scratch(L), (hipStream_t)stream, x, y, batch, ctx_lens, block_tables,
                        max_blocks, max_ctx_len, kv);
}

// The same decode step with its partial results in the library's static
// scratch (no allocation, no event, no synchronisation).
extern "C" tdl_status layer_decode_paged_noalloc(tdl_layer* L, tdl_stream stream, const void* x,
                                                 void* y, int32_t batch, const int32_t* ctx_lens,
                                                 const int32_t* block_tables, int32_t max_blocks,
                                                 int32_t max_ctx_len, tdl_kv_cache* kv) {
  TRY(check_decode(L, x, y, batch, ctx_lens, block_tables, max_blocks, max_ctx_len, kv));
  const tdl_layer_config& c = L->cfg;
  const int H = c.hidden, QD = c.n_q_heads * c.head_dim, I = c.intermediate;
  const int shapes[4][3] = {{L->Nqkv, H, EPI_BIAS_F32}, {H, QD, EPI_RESID_F32},
                            {2 * I, H, EPI_SILU_GATE}, {H, I, EPI_RESID_BF16}};
  size_t g = 0;
  for (int m = 0; m < 4; ++m)
    {
      const int f = gemm_format(L, m, batch);
      g = std::max(g, gemm_plan(batch, shapes[m][0], shapes[m][1], f, shapes[m][2],
                                f != kWDense && L->packed[m]).ws_floats);
    }
  const DecodePlan dp = decode_plan(batch, c.n_q_heads, c.n_kv_heads, c.head_dim, max_ctx_len,
                                    pool_of(L, kv).fmt);
  const size_t g_al = (g + 63) & ~size_t(63);  // partition results start 256-byte aligned
  const size_t need = (g_al + dp.part_floats) * sizeof(float);
  if (need > kStaticScratchBytes)
    return fail(TDL_E_CAPACITY,
                "decode step of batch %d, max_ctx_len %d needs %zu bytes of static scratch; the "
                "maximum is %zu (use layer_decode_paged)",
                batch, max_ctx_len, need, kStaticScratchBytes);
  float* sp = nullptr;
  const hipError_t e = scratch_of(&sp);
  if (e != hipSuccess) return fail(TDL_E_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
  const Scratch sc{sp, g, sp + g_al, dp.part_floats, false};
  return enqueue_decode(L, sc, (hipStream_t)stream, x, y, batch, ctx_lens, block_tables, max_blocks,
                        max_ctx_len, kv);
}

// ---------------------------------------------------------------- stack

struct tdl_stack {
  std::vector<tdl_layer*> layers;  // not owned
  int H = 0;
  int max_rows = 0;
  void* buf[2] = {nullptr, nullptr};  // bf16 [max_rows, H]: activations between layers
  ~tdl_stack() {
    for (void* p : buf)
      if (p) (void)hipFree(p);
  }
};

extern "C" tdl_status stack_create(tdl_layer* const* layers, int32_t n_layers, tdl_stack** out) {
  if (!out) return fail(TDL_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!layers || n_layers < 1) return fail(TDL_E_INVALID, "need n_layers >= 1 layers");
  for (int i = 0; i < n_layers; ++i)
    if (!layers[i]) return fail(TDL_E_INVALID, "layer %d is NULL", i);
  std::unique_ptr<tdl_stack> S(new (std::nothrow) tdl_stack);
  if (!S) return fail(TDL_E_NOMEM, "host allocation failed");
  S->H = layers[0]->cfg.hidden;
  S->max_rows = std::numeric_limits<int>::max();
  for (int i = 0; i < n_layers; ++i) {
    if (layers[i]->cfg.hidden != S->H)
      return fail(TDL_E_INVALID, "layer %d: hidden %d differs from layer 0's %d", i,
                  layers[i]->cfg.hidden, S->H);
    S->max_rows = std::min({S->max_rows, layers[i]->cfg.max_seqs, layers[i]->cfg.max_tokens});
    S->layers.push_back(layers[i]);
  }
  if (n_layers > 1) {
    const size_t bytes = (size_t)S->max_rows * S->H * 2;
    for (void*& p : S->buf)
      if (hipMalloc(&p, bytes) != hipSuccess) {
        p = nullptr;
        (void)hipGetLastError();
        return fail(TDL_E_NOMEM, "hipMalloc of %zu bytes failed", bytes);
      }
  }
  *out = S.release();
  return TDL_OK;
}

extern "C" tdl_status stack_destroy(tdl_stack* stack) {
  delete stack;
  return TDL_OK;
}

extern "C" tdl_status stack_decode_paged(tdl_stack* S, tdl_stream stream, const void* x, void* y,
                                         int32_t batch, const int32_t* ctx_lens,
                                         const int32_t* block_tables, int32_t max_blocks,
                                         int32_t max_ctx_len, tdl_kv_cache* const* kvs) {
  if (!S) return fail(TDL_E_INVALID, "stack is NULL");
  if (!kvs) return fail(TDL_E_INVALID, "kvs is NULL");
  if (batch > S->max_rows)
    return fail(TDL_E_CAPACITY, "batch %d exceeds the stack's %d rows", batch, S->max_rows);
  const int n = (int)S->layers.size();
  auto in_of = [&](int i) { return i == 0 ? x : (const void*)S->buf[(i - 1) & 1]; };
  auto out_of = [&](int i) { return i == n - 1 ? y : S->buf[i & 1]; };
  if (x && y && n > 1 && (x == y)) return fail(TDL_E_INVALID, "y must not alias x");
  // every layer's arguments are checked before the first layer is enqueued
  for (int i = 0; i < n; ++i) {
    const tdl_status st = check_decode(S->layers[i], in_of(i), out_of(i), batch, ctx_lens,
                                       block_tables, max_blocks, max_ctx_len, kvs[i]);
    if (st != TDL_OK) return st;
  }
  for (int i = 0; i < n; ++i)
    TRY(enqueue_decode(S->layers[i], own_scratch(S->layers[i]), (hipStream_t)stream, in_of(i),
                       out_of(i), batch, ctx_lens, block_tables, max_blocks, max_ctx_len, kvs[i]));
  return TDL_OK;
}

extern "C" tdl_status layer_step(tdl_layer* L, tdl_stream stream, const tdl_batch* b, const void* x,
                                 void* y, tdl_kv_cache* kv) {
  if (!L) return fail(TDL_E_INVALID, "layer is NULL");
  if (!b || !x || !y || !kv) return fail(TDL_E_INVALID, "batch, x, y and kv are required");
  if (x == y) return fail(TDL_E_INVALID, "y must not alias x");
  if (((uintptr_t)x | (uintptr_t)y) & 15) return fail(TDL_E_INVALID, "x and y must be 16-byte aligned");
  if (!b->q_start || !b->q_len || !b->ctx_len || !b->block_tables)
    return fail(TDL_E_INVALID, "batch arrays are required");
  if (b->n_seqs < 1 || b->n_prefill_seqs < 0 || b->n_prefill_seqs > b->n_seqs)
    return fail(TDL_E_INVALID, "need 0 <= n_prefill_seqs <= n_seqs, n_seqs >= 1");
  const int n_dec = b->n_seqs - b->n_prefill_seqs;
  if (b->n_rows < b->n_seqs || b->n_rows > L->cfg.max_tokens)
    return fail(b->n_rows < b->n_seqs ? TDL_E_INVALID : TDL_E_CAPACITY,
                "n_rows %d outside [n_seqs, max_tokens=%d]", b->n_rows, L->cfg.max_tokens);
  if (b->n_seqs > L->cfg.max_seqs) return fail(TDL_E_CAPACITY, "n_seqs exceeds max_seqs");
  if (b->n_prefill_seqs > 0 && b->max_q_len < 1)
    return fail(TDL_E_INVALID, "max_q_len must be >= 1 with prefill sequences");
  if (b->max_blocks < 1 || b->max_ctx_len < 1 || b->max_ctx_len > b->max_blocks * 16)
    return fail(TDL_E_INVALID, "max_ctx_len must be in [1, max_blocks*16]");
  if (b->max_ctx_len > L->cfg.max_position)
    return fail(TDL_E_CAPACITY, "max_ctx_len exceeds max_position");
  TRY(check_kv_matches(L, kv));
  hipStream_t st = (hipStream_t)stream;
  if (debug_checks())
    TRY(debug_check_tables(b->ctx_len, b->q_len, b->n_seqs, 1, b->block_tables, b->max_blocks,
                           kv->cfg.n_blocks, b->max_ctx_len, st));
  SeqInfo seq{};
  seq.q_start = b->q_start;
  seq.q_len = b->q_len;
  seq.ctx_len = b->ctx_len;
  seq.n_seqs = b->n_seqs;
  seq.tables = b->block_tables;
  seq.max_blocks = b->max_blocks;
  return run_layer(L, own_scratch(L), st, x, y, b->n_rows, seq, pool_of(L, kv), b->n_prefill_seqs, b->max_q_len,
                   b->n_prefill_seqs, n_dec, b->max_ctx_len);
}

extern "C" tdl_status layer_workspace_view(const tdl_layer* L, tdl_workspace_view* out) {
  if (!L || !out) return fail(TDL_E_INVALID, "NULL argument");
  out->xn = L->xn;
  out->qkv = L->qkv;
  out->q = L->q;
  out->o = L->o;
  out->h = L->h;
  out->hn = L->hn;
  out->a = L->a;
  return TDL_OK;
}

extern "C" tdl_status layer_profile_enable(tdl_layer* L, int enable) {
  if (!L) return fail(TDL_E_INVALID, "layer is NULL");
  for (auto& m : L->prof_pending) {
    (void)hipEventSynchronize(m.b);
    L->prof_free.push_back(m.a);
    L->prof_free.push_back(m.b);
  }
  L->prof_pending.clear();
  for (int i = 0; i < TDL_N_STAGES; ++i) {
    L->prof_ms[i] = 0;
    L->prof_n[i] = 0;
  }
  L->prof_on = enable != 0;
  // events for a few calls made up front: creating them inside a profiled
  // call would hold up its launches
  if (L->prof_on) {
    for (size_t n = L->prof_free.size(); n < 8 * 2 * TDL_N_STAGES; ++n) {
      hipEvent_t e = nullptr;
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) break;
      L->prof_free.push_back(e);
    }
  }
  return TDL_OK;
}

extern "C" tdl_status layer_profile_read(tdl_layer* L, tdl_profile* out) {
  if (!L || !out) return fail(TDL_E_INVALID, "NULL argument");
  for (auto& m : L->prof_pending) {
    HIP_TRY(hipEventSynchronize(m.b));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, m.a, m.b));
    L->prof_ms[m.stage] += ms;
    L->prof_n[m.stage] += 1;
    L->prof_free.push_back(m.a);
    L->prof_free.push_back(m.b);
  }
  L->prof_pending.clear();
  for (int i = 0; i < TDL_N_STAGES; ++i) {
    out->ms[i] = L->prof_ms[i];
    out->launches[i] = L->prof_n[i];
  }
  return TDL_OK;
}

// ============================================================= KV cache

namespace {
bool kv_config_ok(const tdl_kv_config* c) {
  return c && c->n_blocks > 0 && c->block_size == 16 && c->n_kv_heads > 0 &&
         (c->head_dim == 64 || c->head_dim == 128) &&
         (c->kv_dtype == TDL_BF16 || c->kv_dtype == TDL_U8_ASYM || c->kv_dtype == TDL_U4_ASYM) &&
         (c->block_scales == 0 || (c->block_scales == 1 && c->kv_dtype != TDL_BF16));
}
bool kv_coded(const tdl_kv_config* c) {
  return c->kv_dtype == TDL_U8_ASYM || c->kv_dtype == TDL_U4_ASYM;
}
size_t pool_bytes(const tdl_kv_config* c) {
  // bytes per (block, head): 16 tokens x D elements of 2, 1 or 1/2 bytes
  const size_t half_bytes = c->kv_dtype == TDL_BF16 ? 4 : c->kv_dtype == TDL_U8_ASYM ? 2 : 1;
  return align256((size_t)c->n_blocks * c->n_kv_heads * 16 * c->head_dim * half_bytes / 2);
}
size_t param_bytes(const tdl_kv_config* c) {
  return kv_coded(c) ? 4 * align256((size_t)c->n_kv_heads * c->head_dim * 4) : 0;
}
// per-block x per-channel: one exponent byte per (block, head) for K and V
size_t exp_bytes(const tdl_kv_config* c) {
  return c->block_scales ? align256((size_t)c->n_blocks * c->n_kv_heads * 2) : 0;
}
}  // namespace

extern "C" size_t kv_cache_bytes(const tdl_kv_config* cfg) {
  if (!kv_config_ok(cfg)) return 0;
  return 2 * pool_bytes(cfg) + param_bytes(cfg) + exp_bytes(cfg);
}

extern "C" tdl_status kv_cache_alloc(const tdl_kv_config* cfg, void* dev_mem, tdl_kv_cache** out) {
  if (!out) return fail(TDL_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(TDL_E_INVALID, "config is NULL");
  if (cfg->block_size != 16) return fail(TDL_E_UNSUPPORTED, "block_size must be 16");
  if (!kv_config_ok(cfg)) return fail(TDL_E_INVALID, "invalid KV cache configuration");
  if (dev_mem && ((uintptr_t)dev_mem & 255))
    return fail(TDL_E_INVALID, "dev_mem must be 256-byte aligned");
  const size_t bytes = kv_cache_bytes(cfg);
  tdl_kv_cache* kv = new tdl_kv_cache();
  kv->cfg = *cfg;
  if (dev_mem) {
    kv->mem = dev_mem;
  } else {
    if (hipMalloc(&kv->mem, bytes) != hipSuccess) {
      delete kv;
      return fail(TDL_E_NOMEM, "hipMalloc of %zu bytes failed", bytes);
    }
    kv->owned = true;
    hipError_t e = hipMemset(kv->mem, 0, bytes);
    if (e != hipSuccess) {
      (void)hipFree(kv->mem);
      delete kv;
      return fail(TDL_E_HIP, "hipMemset failed: %s", hipGetErrorString(e));
    }
  }
  char* base = (char*)kv->mem;
  kv->k = base;
  kv->v = base + pool_bytes(cfg);
  if (kv_coded(cfg)) {
    char* pb = base + 2 * pool_bytes(cfg);
    const size_t ps = align256((size_t)cfg->n_kv_heads * cfg->head_dim * 4);
    kv->k_scale = (float*)pb;
    kv->k_zp = (int32_t*)(pb + ps);
    kv->v_scale = (float*)(pb + 2 * ps);
    kv->v_zp = (int32_t*)(pb + 3 * ps);
    if (cfg->block_scales) kv->exps = (int8_t*)(pb + param_bytes(cfg));
  }
  // free list: LIFO; blocks come out as 0, 1, 2, ... or in a seeded order
  std::vector<int32_t> order(cfg->n_blocks);
  for (int i = 0; i < cfg->n_blocks; ++i) order[i] = i;
  if (cfg->free_list_seed) {
    uint64_t s = cfg->free_list_seed;
    for (int i = cfg->n_blocks - 1; i > 0; --i) {
      const int j = (int)(splitmix64(s) % (uint64_t)(i + 1));
      std::swap(order[i], order[j]);
    }
  }
  kv->free_list.assign(order.rbegin(), order.rend());
  kv->refs.assign(cfg->n_blocks, 0);
  *out = kv;
  return TDL_OK;
}

extern "C" tdl_status kv_cache_free(tdl_kv_cache* kv) {
  if (!kv) return TDL_OK;
  if (kv->owned) (void)hipFree(kv->mem);
  delete kv;
  return TDL_OK;
}

extern "C" tdl_status kv_cache_view(const tdl_kv_cache* kv, tdl_kv_view* out) {
  if (!kv || !out) return fail(TDL_E_INVALID, "NULL argument");
  const int64_t D = kv->cfg.head_dim, Hkv = kv->cfg.n_kv_heads;
  // u4: strides over bytes, the last index a byte of the row (K) or a
  // channel pair (V)
  const int64_t W = kv->cfg.kv_dtype == TDL_U4_ASYM ? D / 2 : D;
  out->k_pool = kv->k;
  out->v_pool = kv->v;
  out->k_strides[0] = Hkv * 16 * W;
  out->k_strides[1] = 16 * W;
  out->k_strides[2] = W;
  out->k_strides[3] = 1;
  out->v_strides[0] = Hkv * 16 * W;
  out->v_strides[1] = 16 * W;
  out->v_strides[2] = 1;
  out->v_strides[3] = 16;
  out->elem_bytes = kv->cfg.kv_dtype == TDL_BF16 ? 2 : kv->cfg.kv_dtype == TDL_U8_ASYM ? 1 : 0;
  out->k_scale = kv->k_scale;
  out->k_zero_point = kv->k_zp;
  out->v_scale = kv->v_scale;
  out->v_zero_point = kv->v_zp;
  out->block_exp = kv->exps;
  return TDL_OK;
}

extern "C" tdl_status kv_block_table(tdl_kv_cache* kv, int32_t n_seqs, const int32_t* n_tokens,
                                     int32_t max_blocks, int32_t* table) {
  if (!kv || !n_tokens || !table) return fail(TDL_E_INVALID, "NULL argument");
  if (n_seqs < 0 || max_blocks < 1) return fail(TDL_E_INVALID, "n_seqs < 0 or max_blocks < 1");
  size_t need = 0;
  for (int i = 0; i < n_seqs; ++i) {
    if (n_tokens[i] < 0) return fail(TDL_E_INVALID, "n_tokens[%d] < 0", i);
    const int nb = (n_tokens[i] + 15) / 16;
    if (nb > max_blocks)
      return fail(TDL_E_INVALID, "sequence %d needs %d blocks > max_blocks %d", i, nb, max_blocks);
    for (int b = 0; b < nb; ++b) {
      const int32_t e = table[(size_t)i * max_blocks + b];
      if (e < 0) ++need;
      else if (e >= kv->cfg.n_blocks || kv->refs[e] == 0)
        return fail(TDL_E_INVALID, "sequence %d entry %d holds block %d that is not allocated", i,
                    b, e);
    }
  }
  if (need > kv->free_list.size())
    return fail(TDL_E_CAPACITY, "need %zu free blocks, %zu left", need, kv->free_list.size());
  for (int i = 0; i < n_seqs; ++i) {
    const int nb = (n_tokens[i] + 15) / 16;
    for (int b = 0; b < nb; ++b) {
      int32_t& e = table[(size_t)i * max_blocks + b];
      if (e >= 0) continue;
      e = kv->free_list.back();
      kv->free_list.pop_back();
      kv->refs[e] = 1;
    }
  }
  return TDL_OK;
}

namespace {
// Every listed block is allocated, and none is listed more often than it has
// holders (when `holders` is set).
bool check_held(const tdl_kv_cache* kv, const int32_t* blocks, int32_t n, bool holders) {
  std::unordered_map<int32_t, int32_t> times;
  for (int i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (b < 0 || b >= kv->cfg.n_blocks) return fail(TDL_E_INVALID, "block %d out of range", b), false;
    if (kv->refs[b] == 0) return fail(TDL_E_INVALID, "block %d is free", b), false;
    if (holders && ++times[b] > kv->refs[b])
      return fail(TDL_E_INVALID, "block %d released more often than it is held", b), false;
  }
  return true;
}
void drop_hold(tdl_kv_cache* kv, int32_t b) {
  if (--kv->refs[b] == 0) kv->free_list.push_back(b);
}
}  // namespace

extern "C" tdl_status kv_block_release(tdl_kv_cache* kv, const int32_t* blocks, int32_t n) {
  if (!kv || (!blocks && n > 0)) return fail(TDL_E_INVALID, "NULL argument");
  if (n < 0) return fail(TDL_E_INVALID, "n < 0");
  if (!check_held(kv, blocks, n, true)) return TDL_E_INVALID;
  for (int i = 0; i < n; ++i) drop_hold(kv, blocks[i]);
  return TDL_OK;
}

extern "C" tdl_status kv_block_share(tdl_kv_cache* kv, const int32_t* blocks, int32_t n) {
  if (!kv || (!blocks && n > 0)) return fail(TDL_E_INVALID, "NULL argument");
  if (n < 0) return fail(TDL_E_INVALID, "n < 0");
  if (!check_held(kv, blocks, n, false)) return TDL_E_INVALID;
  for (int i = 0; i < n; ++i) ++kv->refs[blocks[i]];
  return TDL_OK;
}

extern "C" int32_t kv_block_refs(const tdl_kv_cache* kv, int32_t block) {
  if (!kv || block < 0 || block >= kv->cfg.n_blocks) return -1;
  return kv->refs[block];
}

extern "C" tdl_status kv_prefix_match(tdl_kv_cache* kv, const uint64_t* keys, int32_t n,
                                      int32_t* blocks, int32_t* n_matched) {
  if (!kv || !n_matched || (n > 0 && (!keys || !blocks))) return fail(TDL_E_INVALID, "NULL argument");
  if (n < 0) return fail(TDL_E_INVALID, "n < 0");
  const uint64_t now = ++kv->tick;
  int32_t m = 0;
  for (; m < n; ++m) {
    auto it = kv->prefix.find(keys[m]);
    if (it == kv->prefix.end()) break;  // the prefix ends at the first miss
    it->second.used = now;
    blocks[m] = it->second.block;
    ++kv->refs[it->second.block];       // the caller now holds it
  }
  *n_matched = m;
  return TDL_OK;
}

extern "C" tdl_status kv_prefix_publish(tdl_kv_cache* kv, const uint64_t* keys,
                                        const int32_t* blocks, int32_t n) {
  if (!kv || (n > 0 && (!keys || !blocks))) return fail(TDL_E_INVALID, "NULL argument");
  if (n < 0) return fail(TDL_E_INVALID, "n < 0");
  if (!check_held(kv, blocks, n, false)) return TDL_E_INVALID;
  std::unordered_map<uint64_t, int32_t> call_block;
  std::unordered_map<int32_t, uint64_t> call_key;
  for (int i = 0; i < n; ++i) {
    auto a = call_block.emplace(keys[i], blocks[i]);
    auto b = call_key.emplace(blocks[i], keys[i]);
    if (a.first->second != blocks[i] || b.first->second != keys[i])
      return fail(TDL_E_INVALID, "entry %d pairs a key or a block of an earlier entry differently", i);
    auto it = kv->prefix.find(keys[i]);
    if (it != kv->prefix.end() && it->second.block != blocks[i]) continue;  // first publisher wins
    auto k = kv->key_of.find(blocks[i]);
    if (k != kv->key_of.end() && k->second != keys[i])
      return fail(TDL_E_INVALID, "block %d is already indexed under another key", blocks[i]);
  }
  const uint64_t now = ++kv->tick;
  for (int i = 0; i < n; ++i) {
    auto it = kv->prefix.find(keys[i]);
    if (it != kv->prefix.end()) {
      if (it->second.block == blocks[i]) it->second.used = now;
      continue;
    }
    kv->prefix.emplace(keys[i], tdl_kv_cache::PrefixEntry{blocks[i], now});
    kv->key_of[blocks[i]] = keys[i];
    ++kv->refs[blocks[i]];  // the index's own hold
  }
  return TDL_OK;
}

extern "C" int32_t kv_prefix_evict(tdl_kv_cache* kv, int32_t n_blocks) {
  if (!kv || n_blocks <= 0) return 0;
  // entries whose block only the index holds, least recently used first
  std::vector<std::pair<uint64_t, uint64_t>> idle;  // (last use, key)
  for (auto& e : kv->prefix)
    if (kv->refs[e.second.block] == 1) idle.push_back({e.second.used, e.first});
  std::sort(idle.begin(), idle.end());
  int32_t done = 0;
  for (auto& u : idle) {
    if (done == n_blocks) break;
    auto it = kv->prefix.find(u.second);
    kv->key_of.erase(it->second.block);
    drop_hold(kv, it->second.block);
    kv->prefix.erase(it);
    ++done;
  }
  return done;
}

extern "C" int32_t kv_prefix_size(const tdl_kv_cache* kv) {
  return kv ? (int32_t)kv->prefix.size() : 0;
}

extern "C" int32_t kv_free_blocks(const tdl_kv_cache* kv) {
  return kv ? (int32_t)kv->free_list.size() : 0;
}

extern "C" tdl_status kv_cache_calibrate(tdl_kv_cache* kv, tdl_stream stream, const float* k,
                                         const float* v, int64_t n_tokens) {
  if (!kv || !k || !v) return fail(TDL_E_INVALID, "NULL argument");
  if (!kv_coded(&kv->cfg)) return fail(TDL_E_INVALID, "cache is not TDL_U8_ASYM or TDL_U4_ASYM");
  if (n_tokens < 1) return fail(TDL_E_INVALID, "n_tokens < 1");
  hipStream_t st = (hipStream_t)stream;
  const int C = kv->cfg.n_kv_heads * kv->cfg.head_dim;
  const int levels = kv->cfg.kv_dtype == TDL_U8_ASYM ? 255 : 15;
  HIP_TRY(tdl::kv_calibrate(k, n_tokens, C, levels, kv->k_scale, kv->k_zp, st));
  HIP_TRY(tdl::kv_calibrate(v, n_tokens, C, levels, kv->v_scale, kv->v_zp, st));
  return TDL_OK;
}

extern "C" tdl_status kv_cache_write(tdl_kv_cache* kv, tdl_stream stream, int32_t n_seqs,
                                     const int32_t* cu_rows, const int32_t* start_pos,
                                     const int32_t* block_tables, int32_t max_blocks,
                                     int32_t src_dtype, const void* k, const void* v,
                                     int32_t n_rows) {
  if (!kv || !cu_rows || !start_pos || !block_tables || !k || !v)
    return fail(TDL_E_INVALID, "NULL argument");
  if (n_seqs < 1 || max_blocks < 1 || n_rows < 0)
    return fail(TDL_E_INVALID, "n_seqs and max_blocks must be >= 1, n_rows >= 0");
  if (src_dtype != TDL_F32 && src_dtype != TDL_BF16)
    return fail(TDL_E_INVALID, "src_dtype must be TDL_F32 or TDL_BF16");
  hipStream_t st = (hipStream_t)stream;
  SeqInfo seq{};
  seq.q_start = cu_rows;
  seq.q_len = nullptr;
  seq.ctx_len = start_pos;
  seq.n_seqs = n_seqs;
  seq.tables = block_tables;
  seq.max_blocks = max_blocks;
  KvPool pool = pool_of(nullptr, kv);
  HIP_TRY(kv_write_rows(k, v, src_dtype == TDL_F32, n_rows, kv->cfg.n_kv_heads, kv->cfg.head_dim,
                        seq, pool, st));
  return TDL_OK;
}

// ============================================================ A8W8 GEMM

extern "C" tdl_status gemm_a8w8(tdl_stream stream, const void* A, const void* B,
                                const float* a_scale, const float* b_scale, int32_t* C_accum,
                                float* out, int32_t M, int32_t N, int32_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(TDL_E_INVALID, "negative size");
  if (M == 0 || N == 0) return TDL_OK;
  if (!A || !B || !a_scale || !b_scale || !out) return fail(TDL_E_INVALID, "NULL argument");
  if (K == 0 || K % 16 != 0) return fail(TDL_E_INVALID, "K must be a positive multiple of 16");
  if (((uintptr_t)A | (uintptr_t)B) & 15) return fail(TDL_E_INVALID, "A and B must be 16-byte aligned");
  HIP_TRY(tdl::a8w8_gemm(A, B, a_scale, b_scale, C_accum, out, M, N, K, (hipStream_t)stream));
  return TDL_OK;
}

// ====================================================== GGUF Q8_0 import

extern "C" tdl_status q80_import_gguf(tdl_stream stream, const void* blocks, int64_t rows, int64_t cols,
                                      void* codes, void* scales) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0)
    return fail(TDL_E_INVALID, "rows >= 0 and a positive multiple of 32 columns required");
  if (rows == 0) return TDL_OK;
  if (!blocks || !codes || !scales) return fail(TDL_E_INVALID, "NULL argument");
  if (((uintptr_t)blocks & 1) || ((uintptr_t)scales & 1) || ((uintptr_t)codes & 15))
    return fail(TDL_E_INVALID, "blocks and scales must be 2-byte aligned, codes 16-byte aligned");
  HIP_TRY(tdl::q80_from_gguf(blocks, rows * (cols / 32), codes, scales, (hipStream_t)stream));
  return TDL_OK;
}

// =============================================================== errors

extern "C" const char* tdl_status_string(tdl_status s) {
  switch (s) {
    case TDL_OK: return "ok";
    case TDL_E_INVALID: return "invalid argument";
    case TDL_E_UNSUPPORTED: return "unsupported";
    case TDL_E_CAPACITY: return "capacity exceeded";
    case TDL_E_NOMEM: return "out of device memory";
    case TDL_E_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" const char* tdl_last_error(void) { return g_last_error.c_str(); }
