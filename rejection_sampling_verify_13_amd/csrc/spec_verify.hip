// spec_verify.hip -- batched draft-verify rejection sampler for MI355X (gfx950).
//
// Method: zwjcode.cn, "生成 4 个 Token 为何不一定要跑 4 次大模型？Speculative
// Decoding 的提议、验证与接受", sections 02-07 (shapes, greedy rule, acceptance
// ratio min(1, p/q), residual normalize(max(0, p - q)), bonus token, identical
// transforms of p and q); pinghaoyang.com.cn, "vLLM 源码完全拆解（十）：投机解码——
// 草稿模型、批量验证与 token 接受流水线", section "拒绝采样：RejectionSampler 的
// 两个分支" with its greedy and random kernel subsections (temperature / top-k /
// top-p preprocessing, -1 placeholders, draft-free residual with the draft
// token's cell removed).  The exact contract is stated in include/spec_verify.h.
//
// Work per call, all on the caller's stream:
//   plan_kernel   (flattened layout, synthetic mode) stores gamma_i and where
//                 the request's rows and drafts sit, clears the outcome bits of
//                 each request's record, and lists the draft rows (request,
//                 position < gamma_i) request-major; in the synthetic
//                 acceptance mode it finds the first rejection A from the
//                 uniforms and lists row A alone.  The padded layout in the
//                 standard mode needs no plan: each row workgroup finds gamma_i
//                 from the request's ids (one load per lane) and the request's
//                 outcome is read back from its rows' records.
//   row_kernel    one 256-thread workgroup per real row: the draft rows, then
//                 (standard mode) one bonus row per request.  It streams the target-logit
//                 row and, at draft positions of sampled requests, the
//                 draft-probability row once (16-byte nontemporal loads,
//                 several steps of loads in flight while the current step is
//                 reduced).
//                 Without top-k: row max, sum of exp over the row (fp32 terms,
//                 fp64 accumulation), sum of q^(1/T), draft-row validity.
//                 With top-k (k <= kKFast): row max and validity only, plus
//                 per wave an LDS buffer of the 8-token chunks whose largest
//                 value reaches a rising threshold that never exceeds the row's
//                 k-th largest value, so one pass yields every top-k token; one
//                 wave per distribution then finds the exact k-th largest, the
//                 fp64 kept masses and the top-p cut from LDS.  Other filter
//                 settings use a radix select that re-reads the row.  Greedy
//                 rows take the argmax.  p'(y) and q'(y) are evaluated in fp64
//                 and the flag u * q'(y) < p'(y) stored; a row that may be the
//                 one drawn from (the bonus row, or a rejected draft row) with
//                 its top-k set in LDS also draws its token there.  Each row
//                 writes its accept bit, fault bits and draw to its own record
//                 (and, with a plan, ORs them into the request's record).
//   draw_kernel   per request whose row A made no draw of its own: the sums
//                 of row A's draw weights per 512-token block, the row spread
//                 over workgroups of kDrawSpan steps.
//   find_kernel   per request: the first rejection A from the record, the
//                 outputs (-1 padded), and, where row A made no draw of its
//                 own, the draw by inverse CDF over ascending token id from
//                 the block sums (one scan over all of them, then the
//                 crossing block re-read).
//   finish_kernel (instead of the two above, for calls without token lists
//                 and with 128 to 384 requests) one 512-thread workgroup per
//                 request: the outputs, row A's block sums in LDS, the search.
//   rollback_kernel  (own entry point, after a verify call) the KV bookkeeping
//                 of the rejected drafts.
//
// Token lists (flattened entry point with options): the row and draw kernels
// have instantiations that copy the request's banned tokens, and the
// position's repetition-penalty list, into LDS and rewrite each step's raw
// values as they arrive (a banned token: -inf / 0; a penalised one: the rule
// of include/spec_verify.h), so every later step sees the transformed row;
// the instantiation without lists is the one the plain entry points use.

// Compile: hipcc --offload-arch=gfx950 -O3 -shared -fPIC
//          -Xclang -target-feature -Xclang -packed-fp32-ops

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "spec_verify.h"

namespace {

constexpr int kBlock = 256;             // threads per workgroup (4 waves)
constexpr int kWaves = kBlock / 64;
constexpr int kCh = 8;                  // tokens per thread per step
constexpr int kStep = kBlock * kCh;     // tokens per workgroup step (2048)
constexpr int kCap = 160;               // buffered candidate chunks per wave and distribution
constexpr int kKFast = 64;              // largest top_k served by the candidate buffers
constexpr int kSeg = 128;               // gathered candidate tokens per wave and distribution (LDS)
constexpr int kDrawSpan = 4;            // draw pass: 2048-token steps per workgroup
constexpr int kDrawWin = 4;             // draw pass: steps in flight per workgroup
constexpr int kFindPer = 8;             // draw search: block sums per lane and load round
constexpr int kFinBlock = 512;          // fused draw pass: threads per workgroup (one workgroup per request)
constexpr int kFinWaves = kFinBlock / 64;
constexpr int kFinWin = 4;              // fused draw pass: 512-token blocks in flight per wave
constexpr int kFinMinN = 128;           // fused draw pass from this many requests (half the CUs) ...
constexpr int kFinMaxN = 384;           // ... to this many (1.5 per CU): one request per workgroup
                                        // balances the draws left to the pass only in that range
constexpr int kMaxGamma = 64;

enum {
  kFaultDraftId = SPEC_VERIFY_FAULT_DRAFT_ID,
  kFaultTemperature = SPEC_VERIFY_FAULT_TEMPERATURE,
  kFaultTopP = SPEC_VERIFY_FAULT_TOP_P,
  kFaultTargetRow = SPEC_VERIFY_FAULT_TARGET_ROW,
  kFaultDraftRow = SPEC_VERIFY_FAULT_DRAFT_ROW,
  kFaultDraftMass = SPEC_VERIFY_FAULT_DRAFT_MASS,
  kFaultDraftCount = SPEC_VERIFY_FAULT_DRAFT_COUNT,
  kFaultBanList = SPEC_VERIFY_FAULT_BAN_LIST,
  kFaultRowIndex = SPEC_VERIFY_FAULT_ROW_INDEX,
  kFaultPenalty = SPEC_VERIFY_FAULT_PENALTY,
};
constexpr int kBanMax = 512;            // banned tokens per request (ascending list kept in LDS)
constexpr int kPenMax = 1024;           // penalised tokens per row (ascending list kept in LDS)

// Per-row results (64 bytes).
struct RowStats {
  float m;        // max logit of the row
  float cut_p;    // target token kept iff logit >= cut_p
  float cut_q;    // draft token kept iff q >= cut_q
  union {
    int argmax;   // greedy rows: lowest id of the max logit
    float qinv;   // stochastic rows: 1 / qs, the scale of the tempered draft weights (q / qs)^(1/T)
  };
  double z;       // sum over the kept set of 2^((l - m) * c), c = log2(e) / T in fp32
  double r;       // sum over the kept set of (q / qs)^(1/T) (of q at T = 1)
  double p_y;     // p'(y) at a draft position
  double q_y;     // q'(y) at a draft position
  double s;       // mass S of the draw made in the row (when draw >= 0)
  int flags;      // bit 0: accepted; bits 8..15: fault bits
  int draw;       // token drawn from this row's draw weights, -1: not drawn in the row pass
};
static_assert(sizeof(RowStats) == 64, "RowStats layout");

// One request's place in the inputs and the outcome of its rows.  The plan
// kernel writes the layout fields and clears the bits; each row workgroup ORs
// its own bits in; the draw pass reads the record once to find the first
// rejection A.
struct ReqRec {
  unsigned long long acc;     // bit j: the draft token at position j was accepted
  unsigned long long nodraw;  // bit j: row j (j < 64) made no draw of its own
  unsigned int nodraw64;      // 1: row 64 (gamma_i = 64) made no draw of its own
  unsigned int fault;         // fault bits of the request's rows (row pass)
  int gamma;                  // gamma_i
  int tgt0;                   // target_logits row of position 0
  int id0;                    // index of draft 0 in draft_ids and u_accept
  int q0;                     // draft_probs row of position 0; -1: no draft rows
  unsigned int lfault;        // layout fault found by the plan kernel
  int pad;
};
static_assert(sizeof(ReqRec) == 48, "ReqRec layout");

// Sum of the draw weights w of one 512-token block (one wave's tokens of one
// step) of row A.
struct DrawSum {
  double sw;
};
static_assert(sizeof(DrawSum) == 8, "DrawSum layout");

struct Args {
  int N, G, V;
  const int32_t* ids;
  const float* q;
  const void* logits;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* u_accept;
  const float* u_sample;
  int32_t* out_tokens;
  int32_t* out_num;
  double* d_py;
  double* d_qy;
  double* d_resid;
  int32_t* d_fault;
  RowStats* stats;
  ReqRec* rec;          // per request
  DrawSum* dsum;        // [N][steps][kWaves]
  unsigned int* nfault; // faulted requests of this call (workspace head; cleared by the plan kernel)
  int* plan;            // [0]: number of listed rows D; then D entries i * 128 + j, request-major
  int dparts;           // draw pass: workgroups per request (kDrawSpan steps each)
  // flattened layout (cu == nullptr: the padded [N, G] layout)
  const int32_t* cu;    // [N] inclusive prefix sums of gamma_i
  const uint8_t* has_q; // [N] request i has draft rows iff nonzero; nullptr: all do (when q != nullptr)
  int T;                // number of drafts, cu[N - 1]
  const int32_t* bidx;  // [N] target_logits row of each bonus position, or nullptr (rows in request order)
  const int32_t* tidx;  // [T] target_logits row of each draft position (with bidx)
  int R;                // rows of target_logits (with bidx)
  const int32_t* ban_off;  // [N + 1] banned-token list offsets, or nullptr
  const int32_t* ban_ids;  // ascending ids per request; nullptr when every list is empty
  const int32_t* pen_off;  // [T + N + 1] penalty list offsets per position, or nullptr
  const int32_t* pen_ids;  // ascending ids per position; nullptr when every list is empty
  const int32_t* pen_cnt;  // their counts in the generated output
  const float* pen_rep;    // [N] repetition penalty, or nullptr (1)
  const float* pen_pres;   // [N] presence penalty, or nullptr (0)
  const float* pen_freq;   // [N] frequency penalty, or nullptr (0)
  int dslots;           // direct mode: row-pass blocks per request for its draft positions
  int direct;           // 1: padded layout, standard mode: no plan kernel; each row workgroup finds
                        // gamma_i from the ids and the outcome lives in the rows' records
  int synthetic;        // 1: the synthetic acceptance mode (draft j accepted iff u_j < srates[j])
  const float* srates;  // synthetic acceptance rates [G]
};

// Direct mode: row-pass blocks per request for its draft positions (gmax,
// one more when gmax is a multiple of 8, so that a request's positions do
// not each land on one XCD), and the row pass's grid.
__host__ __device__ inline int direct_slots(int G) { return (G > 0 && G % 8 == 0) ? G + 1 : G; }
__host__ __device__ inline long long row_blocks(int N, int G, bool synthetic, bool direct) {
  if (synthetic) return N;  // row A only
  return (long long)N * ((direct ? direct_slots(G) : G) + 1);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row data is read through global-address-space pointers so that loads are
// global (not flat) instructions: they then count only against the vector
// memory counter and the next step's loads stay in flight across LDS work.
#define GLOBAL_AS __attribute__((address_space(1)))
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))
template <class T>
__device__ inline const GLOBAL_AS T* gptr(const T* p) {
  return (const GLOBAL_AS T*)p;
}

// ------------------------------------------------------------------------------------------
// element access: one "step" is 8 consecutive tokens of a lane, kept raw until reduced
// ------------------------------------------------------------------------------------------

struct Bf16 {
  typedef uint16_t T;
  struct Raw {
    u32x4 a;
  };
  __device__ static float at(const uint16_t* p, size_t x) { return __uint_as_float((uint32_t)gptr(p)[x] << 16); }
  __device__ static Raw load(const uint16_t* p) {
    Raw r;
    r.a = __builtin_nontemporal_load(gptr(reinterpret_cast<const u32x4*>(p)));
    return r;
  }
  // tokens at or past V read as -inf
  __device__ static Raw gather(const uint16_t* p, int base, int V) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t lo = (base + 2 * t < V) ? (uint32_t)gptr(p)[base + 2 * t] : 0xff80u;
      const uint32_t hi = (base + 2 * t + 1 < V) ? (uint32_t)gptr(p)[base + 2 * t + 1] : 0xff80u;
      w[t] = lo | (hi << 16);
    }
    Raw r;
    r.a = u32x4{w[0], w[1], w[2], w[3]};
    return r;
  }
  __device__ static void unpack(const Raw& r, float v[8]) {
    v[0] = __uint_as_float(r.a.x << 16); v[1] = __uint_as_float(r.a.x & 0xffff0000u);
    v[2] = __uint_as_float(r.a.y << 16); v[3] = __uint_as_float(r.a.y & 0xffff0000u);
    v[4] = __uint_as_float(r.a.z << 16); v[5] = __uint_as_float(r.a.z & 0xffff0000u);
    v[6] = __uint_as_float(r.a.w << 16); v[7] = __uint_as_float(r.a.w & 0xffff0000u);
  }
};

struct F32 {
  typedef float T;
  struct Raw {
    u32x4 a, b;
  };
  __device__ static float at(const float* p, size_t x) { return gptr(p)[x]; }
  __device__ static Raw load(const float* p) {
    Raw r;
    r.a = __builtin_nontemporal_load(gptr(reinterpret_cast<const u32x4*>(p)));
    r.b = __builtin_nontemporal_load(gptr(reinterpret_cast<const u32x4*>(p)) + 1);
    return r;
  }
  // tokens at or past V read as `fill` (-inf for logits, 0 for probabilities)
  __device__ static Raw gather(const float* p, int base, int V, uint32_t fill) {
    uint32_t w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) w[t] = (base + t < V) ? __float_as_uint(gptr(p)[base + t]) : fill;
    Raw r;
    r.a = u32x4{w[0], w[1], w[2], w[3]};
    r.b = u32x4{w[4], w[5], w[6], w[7]};
    return r;
  }
  __device__ static Raw gather(const float* p, int base, int V) { return gather(p, base, V, 0xff800000u); }
  __device__ static void unpack(const Raw& r, float v[8]) {
    v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y); v[2] = __uint_as_float(r.a.z);
    v[3] = __uint_as_float(r.a.w); v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
    v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
  }
  __device__ static void bits(const Raw& r, uint32_t u[8]) {
    u[0] = r.a.x; u[1] = r.a.y; u[2] = r.a.z; u[3] = r.a.w;
    u[4] = r.b.x; u[5] = r.b.y; u[6] = r.b.z; u[7] = r.b.w;
  }
};

// One step of logits: vector load when every row start is 16-byte aligned
// (the tail step masks tokens past V to -inf), scalar loads otherwise.
template <class LT, bool VEC>
__device__ inline typename LT::Raw load_logits(const typename LT::T* row, int base, int V) {
  if (VEC && base + kCh <= V) return LT::load(row + base);
  return LT::gather(row, base, V);
}
template <bool VEC>
__device__ inline F32::Raw load_probs(const float* row, int base, int V) {
  if (VEC && base + kCh <= V) return F32::load(row + base);
  return F32::gather(row, base, V, 0u);
}

// order-preserving 32-bit key of a float; -0 and +0 share a key
__device__ inline uint32_t okey(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float okey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// 3-input max without canonicalising the operands (NaN operands are ignored
// unless all are NaN; NaN rows are caught through the exponential sums).
__device__ inline float fmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float max8(const float v[8]) {
  return fmax3(fmax3(v[0], v[1], v[2]), fmax3(v[3], v[4], v[5]), fmax3(v[6], v[7], v[7]));
}
__device__ inline uint32_t max8u(const uint32_t u[8]) {
  return max(max(max(u[0], u[1]), max(u[2], u[3])), max(max(u[4], u[5]), max(u[6], u[7])));
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Tempered draft weights are (q / qs)^(1/T) with qs = 2^(E - 126), E the
// biased fp32 exponent of the row's largest q clamped to [1, 252]: the power
// of two just above that q.  The factor qs^(-1/T) is common to every weight
// and to their sum, so q' is unchanged, while q / qs is exact, the weights stay
// within [0, 1] and the fp32 exponent log2(q / qs) / T stays small for the
// tokens that carry the mass (at low T, log2(q) / T itself reaches hundreds,
// where one fp32 ulp is ~1e-5).  Rows whose largest q is subnormal or above
// 2^126 lie outside that scheme (the first read as zero mass).
__device__ inline int scale_e(uint32_t qmax_bits) { return min(max((int)(qmax_bits >> 23), 1), 252); }
__device__ inline float scale_inv(int e) { return __uint_as_float((uint32_t)(253 - e) << 23); }
// An exponent scale (c = log2(e) / T for the target, 1 / T for the draft) in
// fp64 and as an fp32 pair hi + lo with hi strictly below the value, so lo > 0.
// A streamed exponent d * c is then fma(d, hi, d * lo): the exact product
// rounded about once.  Rounding c itself to fp32 would instead scale every
// exponent by the same relative error (up to 6e-8), a bias proportional to
// the exponent that does not cancel in the normalised weights.  With lo > 0,
// d = -inf gives -inf (weight 0) and NaN stays NaN.
struct Scale2 {
  double d;
  float hi, lo;
};
__device__ inline Scale2 scale2(double v) {
  Scale2 s;
  s.d = v;
  s.hi = (float)v;
  if ((double)s.hi >= v) s.hi = __uint_as_float(__float_as_uint(s.hi) - 1u);  // v > 0
  s.lo = (float)(v - (double)s.hi);
  return s;
}
__device__ inline float smul(float x, const Scale2& s) { return __builtin_fmaf(x, s.hi, x * s.lo); }
__device__ inline Scale2 target_scale(float T) { return scale2(1.4426950408889634 / (double)T); }
__device__ inline Scale2 draft_scale(float T) { return scale2(1.0 / (double)T); }

// (qs(e0) / qs(e1))^(1/T), e0 <= e1: in fp64 where wave and block sums are
// combined; inside the streaming loop (a thread's running sum meeting a q in
// a higher binade, a few times per row) the exponent is rounded once and the
// power formed in fp32
__device__ inline double scale_step(int e0, int e1, const Scale2& invT) {
  return exp2((double)(e0 - e1) * invT.d);
}
__device__ inline double scale_step32(int e0, int e1, const Scale2& invT) {
  return (double)fast_exp2(smul((float)(e0 - e1), invT));
}
// the weight in fp64, the same expression wherever a single value is needed
// (qinv = 1 / qs is a power of two: the product is exact)
__device__ inline double temper_q(float q, float T, float qinv) {
  return T == 1.f ? (double)q : pow((double)q * (double)qinv, 1.0 / (double)T);
}
// The streamed tempered weight.  In fp32 the exponent log2(q / qs) / T carries
// the hardware log2's error (about 6e-8 absolute) times 1/T, and is rounded to
// fp32: at T = 0.05 a weight near the row's largest is off by ~1e-6.  So when
// 1/T exceeds kPreciseInvT, the weights that can carry mass are formed in fp64
// instead: those whose fp32 exponent is above thr = -(1/T + 24).  The largest
// weight is at least 2^(-1/T) (qs is within a factor 2 of the largest q), so
// the tokens left in fp32 each weigh under 2^-24 of it.
constexpr double kPreciseInvT = 2.0;
struct DraftW {
  Scale2 invT;
  float thr;      // exponent above which the weight is formed in fp64
  bool precise;   // 1/T > kPreciseInvT
};
__device__ inline DraftW draft_w(float T) {
  DraftW w;
  w.invT = draft_scale(T);
  w.precise = w.invT.d > kPreciseInvT;
  w.thr = -(float)(w.invT.d + 24.0);
  return w;
}
// r^(1/T) in fp64 for a positive float r (r = q / qs, exact), to about 1e-13
// relative, in straight-line code (no library call).  r = m 2^E with
// m in [sqrt(1/2), sqrt(2)); log2(m) = (2 / ln 2) atanh(t), t = (m - 1) / (m + 1),
// |t| < 0.1716, from the series t + t^3/3 + ... + t^17/17; then x = (E +
// log2 m) / T = n + f with n an integer and |f| <= 1/2, and 2^f = e^(f ln 2)
// from its Taylor series to the 13th power.
__device__ inline double precise_weight(float r, double invT) {
  int E;
  double m = 2.0 * (double)frexpf(r, &E);  // r = m 2^(E - 1), m in [1, 2)
  E -= 1;
  if (m > 1.4142135623730951) {
    m *= 0.5;
    E += 1;
  }
  const double t = (m - 1.0) / (m + 1.0), t2 = t * t;
  double a = 1.0 / 17;
  a = fma(a, t2, 1.0 / 15);
  a = fma(a, t2, 1.0 / 13);
  a = fma(a, t2, 1.0 / 11);
  a = fma(a, t2, 1.0 / 9);
  a = fma(a, t2, 1.0 / 7);
  a = fma(a, t2, 1.0 / 5);
  a = fma(a, t2, 1.0 / 3);
  a = fma(a, t2, 1.0);
  const double x = ((double)E + 2.8853900817779268 * t * a) * invT;  // 2 / ln 2
  const double n = fmax(rint(x), -2000.0);
  const double f = (x - n) * 0.6931471805599453;  // ln 2
  double e = 1.0 / 6227020800.0;                 // 1 / 13!
  e = fma(e, f, 1.0 / 479001600.0);
  e = fma(e, f, 1.0 / 39916800.0);
  e = fma(e, f, 1.0 / 3628800.0);
  e = fma(e, f, 1.0 / 362880.0);
  e = fma(e, f, 1.0 / 40320.0);
  e = fma(e, f, 1.0 / 5040.0);
  e = fma(e, f, 1.0 / 720.0);
  e = fma(e, f, 1.0 / 120.0);
  e = fma(e, f, 1.0 / 24.0);
  e = fma(e, f, 1.0 / 6.0);
  e = fma(e, f, 0.5);
  e = fma(e, f, 1.0);
  e = fma(e, f, 1.0);
  return ldexp(e, (int)n);
}
// The same, out of line: the streaming loops and the draw pass call it from
// rarely taken branches, and keep their registers (inlined there, its fp64
// temporaries made the row kernel spill in its hot loops).
__device__ __noinline__ double precise_weight_call(float r, double invT) { return precise_weight(r, invT); }
// fp32 weight of q with qinv = 1 / qs, or (precise tokens) 0 with the fp64
// weight added to acc
__device__ inline float temper_w32(float q, const DraftW& dw, float qinv, double& acc) {
  const float r = q * qinv;
  const float x = smul(fast_log2(r), dw.invT);
  if (dw.precise && x > dw.thr) {
    acc += precise_weight_call(r, dw.invT.d);
    return 0.f;
  }
  return fast_exp2(x);
}
__device__ inline double temper_w64(float q, const DraftW& dw, float qinv) {
  const float r = q * qinv;
  const float x = smul(fast_log2(r), dw.invT);
  if (dw.precise && x > dw.thr) return precise_weight_call(r, dw.invT.d);
  return (double)fast_exp2(x);
}
// streamed target weight 2^((l - m) * c); the largest is 1, so a token's
// absolute error stays near 2^x * |x| * 2^-25, small wherever 2^x is not
__device__ inline float mass_p32(float l, float m, const Scale2& c) { return fast_exp2(smul(l - m, c)); }
// 2^((l - m) * c) in fp64
__device__ inline double mass_p(float l, float m, const Scale2& c) {
  return exp2(((double)l - (double)m) * c.d);
}

// ------------------------------------------------------------------------------------------
// per-row records
//
// A row's record is written by its own workgroup and read only by later
// launches on the same stream (the draw and find kernels): the end of one
// kernel and the start of the next order the writes before the reads, so the
// records are plain stores and no workgroup waits on another within a launch.
// ------------------------------------------------------------------------------------------

template <class T>
__device__ inline void publish(T* dst, const T& v) {
  static_assert(sizeof(T) % 8 == 0, "records are whole 8-byte words");
  const uint64_t* src = reinterpret_cast<const uint64_t*>(&v);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
  for (int t = 0; t < (int)(sizeof(T) / 8); ++t) d[t] = src[t];
}

// Adds row j's outcome to request i's record (one thread; plan mode).  The
// ORs return nothing, so the workgroup does not wait for them; the draw
// pass, a later launch, reads the record.
__device__ inline void note_row(const Args& a, int i, int j, int acc, int fault, bool nodraw) {
  if (a.direct) return;  // direct mode: the row's own record carries the outcome
  ReqRec* r = a.rec + i;
  if (acc) __hip_atomic_fetch_or(&r->acc, 1ull << j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (fault) __hip_atomic_fetch_or(&r->fault, (unsigned int)fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (nodraw) {
    if (j < 64) __hip_atomic_fetch_or(&r->nodraw, 1ull << j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else __hip_atomic_fetch_or(&r->nodraw64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------------------------------
// wave / block helpers
// ------------------------------------------------------------------------------------------

__device__ inline int lane_id() { return threadIdx.x & 63; }
// Wave-uniform copies (s_readfirstlane): values that are the same in every
// lane but reach a function through VGPR arguments or LDS, so that the
// compiler keeps them in scalar registers and branches on them with scalar
// branches instead of exec masks.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ inline float uni(float x) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x))); }
__device__ inline double uni(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <class T>
__device__ inline T* uni(T* p) {
  const uint64_t b = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// set bits of m below this lane (v_mbcnt: no mask register kept live)
__device__ inline int mbcnt(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ inline int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// Unsigned max / min over a full wave with DPP lane moves (no LDS round
// trips): butterflies inside each row of 16 lanes, then the row broadcasts;
// lane 63 ends with the result.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_mov<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_mov<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_mov<0x141, 0xF>(v));  // row_half_mirror
  v = max(v, dpp_mov<0x140, 0xF>(v));  // row_mirror
  v = max(v, dpp_mov<0x142, 0xA>(v));  // row_bcast:15
  v = max(v, dpp_mov<0x143, 0xC>(v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_mov<0xB1, 0xF>(v));
  v = min(v, dpp_mov<0x4E, 0xF>(v));
  v = min(v, dpp_mov<0x141, 0xF>(v));
  v = min(v, dpp_mov<0x140, 0xF>(v));
  v = min(v, dpp_mov<0x142, 0xA>(v));
  v = min(v, dpp_mov<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Full-wave float max and fp64 sum with DPP (every lane must be active);
// lanes of rows outside a row_bcast mask add the identity.
__device__ inline float wave_max_f32(float v) {
  v = __builtin_fmaxf(v, __uint_as_float(dpp_mov<0xB1, 0xF>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(dpp_mov<0x4E, 0xF>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(dpp_mov<0x141, 0xF>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(dpp_mov<0x140, 0xF>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(dpp_mov<0x142, 0xA>(__float_as_uint(v))));
  v = __builtin_fmaxf(v, __uint_as_float(dpp_mov<0x143, 0xC>(__float_as_uint(v))));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <int CTRL, int ROWS>
__device__ inline double dpp_add_src(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ inline double wave_sum_f64(double v) {
  v += dpp_add_src<0xB1, 0xF>(v);
  v += dpp_add_src<0x4E, 0xF>(v);
  v += dpp_add_src<0x141, 0xF>(v);
  v += dpp_add_src<0x140, 0xF>(v);
  v += dpp_add_src<0x142, 0xA>(v);
  v += dpp_add_src<0x143, 0xC>(v);
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over a full wave (row shifts, then row broadcasts).
template <int CTRL, int ROWS>
__device__ inline int dpp_src0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ inline int wave_incl_scan_i32(int v) {
  v += dpp_src0<0x111, 0xF>(v);  // row_shr:1
  v += dpp_src0<0x112, 0xF>(v);  // row_shr:2
  v += dpp_src0<0x114, 0xF>(v);  // row_shr:4
  v += dpp_src0<0x118, 0xF>(v);  // row_shr:8
  v += dpp_src0<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_src0<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

__device__ inline double readlane_d(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Block reductions: wave butterflies, then the four wave results combined in a
// fixed order, so every thread gets the same, run-to-run reproducible value.
__device__ inline double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}
__device__ inline float block_max_f(float v, float* red) {
  v = wave_max_f(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ inline int block_max_i(int v, int* red) {
  v = wave_max_i(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ inline int block_min_i(int v, int* red) {
  v = wave_min_i(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = min(min(red[0], red[1]), min(red[2], red[3]));
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------------------------------
// request parameters
// ------------------------------------------------------------------------------------------

// wave-uniform copies (scalar registers) of scale pairs and draft-weight settings
__device__ inline Scale2 uni_s2(Scale2 v) {
  v.d = uni(v.d);
  v.hi = uni(v.hi);
  v.lo = uni(v.lo);
  return v;
}
__device__ inline DraftW uni_dw(DraftW d) {
  d.invT = uni_s2(d.invT);
  d.thr = uni(d.thr);
  d.precise = uni((int)d.precise);
  return d;
}

struct Req {
  int gamma;      // number of draft tokens
  int tgt0;       // target_logits row of position 0 (rows in request order)
  long long trow; // target_logits row of the row being processed (row kernel)
  int id0;        // index of draft 0 in draft_ids and u_accept
  int q0;         // draft_probs row of position 0; -1: no draft rows
  float T;        // temperature
  int k;          // top_k (raw)
  float p;        // top_p (raw)
  int fault;      // parameter faults
  bool greedy;
  bool kact;      // top-k filter active
  bool pact;      // top-p filter active
};

// The request's layout and parameters, and the draft-id check; every wave of
// the block evaluates this redundantly (gamma_i <= 64 ids).  Plan mode: the
// layout from the plan kernel's record.  Direct mode (padded layout): gamma_i
// is the index of the first negative id, found from one load per lane, and
// the rest follows from i; the parameters load alongside.
__device__ inline Req load_req(const Args& a, int i) {
  Req r;
  const int lane = lane_id();
  r.T = a.temperature ? a.temperature[i] : 1.f;
  r.k = a.top_k ? a.top_k[i] : 0;
  r.p = a.top_p ? a.top_p[i] : 1.f;
  int id;
  if (a.direct) {
    r.tgt0 = i * (a.G + 1);
    r.id0 = i * a.G;
    r.q0 = a.q ? i * a.G : -1;
    r.fault = 0;
    id = lane < a.G ? a.ids[(size_t)r.id0 + lane] : 0;
    const uint64_t neg = __ballot(lane < a.G && id < 0);
    r.gamma = neg ? __ffsll((unsigned long long)neg) - 1 : a.G;
  } else {
    const ReqRec* rr = a.rec + i;
    r.gamma = rr->gamma;
    r.tgt0 = rr->tgt0;
    r.id0 = rr->id0;
    r.q0 = rr->q0;
    r.fault = (int)rr->lfault;
    id = lane < r.gamma ? a.ids[(size_t)r.id0 + lane] : 0;
  }
  if (__ballot(lane < r.gamma && (id < 0 || id >= a.V))) r.fault |= kFaultDraftId;
  const float T = r.T;
  if (isnan(T) || T < 0.f || isinf(T) || (T > 0.f && T < FLT_MIN)) r.fault |= kFaultTemperature;
  r.greedy = (T == 0.f);
  if (!r.greedy && !(r.fault & kFaultTemperature) && (isnan(r.p) || r.p <= 0.f)) r.fault |= kFaultTopP;
  r.kact = r.k >= 1 && r.k < a.V;
  r.pact = r.p < 1.f;
  return r;
}

// ------------------------------------------------------------------------------------------
// candidate chunk buffers for top-k (rising threshold)
// ------------------------------------------------------------------------------------------

// Candidate chunks of one wave for one distribution.  A chunk is the 8
// consecutive tokens one lane holds in one step: its largest order key, its
// first token id and its raw values (R: the step's raw load), so that the
// kept set is later found from LDS alone.  A chunk is appended when its key
// reaches the wave's threshold; when the buffer fills, the threshold is raised
// to the k-th largest buffered key and the buffer compacted.  The threshold
// never exceeds the k-th largest value among the tokens the wave has seen, so
// after the pass the buffer holds every one of the wave's tokens at or above
// the row's k-th largest value.
template <class R>
struct ChunkBuf {
  uint32_t key[kCap];
  int base[kCap];
  R val[kCap];
};

// Wave-uniform state of one buffer.
struct ChunkState {
  int cnt;
  uint32_t thr;   // chunks whose key is below it are not buffered
  int ovf;        // ties kept the buffer too full: the radix select decides
};

constexpr int kCapLane = (kCap + 63) / 64;
constexpr int kSlack = 16;             // refresh stops once at most k + kSlack chunks stay

// member-wise copies of raw steps to and from LDS
__device__ inline void raw_put(LDS_AS Bf16::Raw* d, const Bf16::Raw& r) { d->a = r.a; }
__device__ inline void raw_put(LDS_AS F32::Raw* d, const F32::Raw& r) { d->a = r.a; d->b = r.b; }
__device__ inline void raw_get(const LDS_AS Bf16::Raw* s, Bf16::Raw& r) { r.a = s->a; }
__device__ inline void raw_get(const LDS_AS F32::Raw* s, F32::Raw& r) { r.a = s->a; r.b = s->b; }

// Raise the threshold and keep only the chunks at or above it.  The new
// threshold T has at least k buffered chunk keys >= T (so it does not exceed
// the k-th largest chunk key, a lower bound of the wave's k-th largest value)
// and, unless ties prevent it, at most k + slack: bisection on the key bits
// below the common prefix of the smallest and largest key, stopping as soon
// as the count is within that band.  Plain values in and out, so callers keep
// their state in registers.
template <class R>
__device__ __forceinline__ ChunkState chunk_refresh(LDS_AS ChunkBuf<R>* b, ChunkState s, int k, int slack) {
  // the wave's next loads wait on this: issue ahead of the streaming waves
  __builtin_amdgcn_s_setprio(2);
  const int lane = lane_id();
  s.cnt = uni(s.cnt);
  s.ovf = uni(s.ovf);
  k = uni(k);
  slack = uni(slack);
  uint32_t key[kCapLane];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int t = 0; t < kCapLane; ++t) {
    const bool h = lane + 64 * t < s.cnt;
    key[t] = h ? b->key[lane + 64 * t] : 0u;
    if (h) {
      kmax = max(kmax, key[t]);
      kmin = min(kmin, key[t]);
    }
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  uint32_t thr = kmin;
  if (kmin != kmax) {
    const int top = 31 - __clz((int)(kmin ^ kmax));
    thr = kmin & ~((2u << top) - 1u);
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t T = thr | (1u << bit);
      int c = 0;
#pragma unroll
      for (int t = 0; t < kCapLane; ++t) c += __popcll(__ballot(key[t] >= T));
      if (c >= k) {
        thr = T;
        if (c <= k + slack) break;
      }
    }
  }
  int n = 0;
  // compaction in slot order: an entry only moves to a lower slot, and slot
  // group t is read completely before any of it is overwritten
#pragma unroll
  for (int t = 0; t < kCapLane; ++t) {
    const int e = lane + 64 * t;
    const bool h = e < s.cnt;
    const int base = h ? b->base[e] : 0;
    R val{};
    if (h) raw_get(&b->val[e], val);
    wave_lds_sync();
    const bool keep = h && key[t] >= thr;
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int p = n + mbcnt(m);
      b->key[p] = key[t];
      b->base[p] = base;
      raw_put(&b->val[p], val);
    }
    n += __popcll(m);
    wave_lds_sync();
  }
  s.cnt = n;
  s.thr = thr;
  if (s.cnt > kCap - 64) s.ovf = 1;
  __builtin_amdgcn_s_setprio(0);
  return s;
}

// Offer this lane's chunk (largest key `key`, first token `base`, raw values).
template <class R>
__device__ inline void chunk_offer(LDS_AS ChunkBuf<R>* b, ChunkState& s, int k, bool valid, uint32_t key, int base,
                                   const R& raw) {
  bool ins = valid && key >= s.thr;
  uint64_t m = __ballot(ins);
  if (!m || s.ovf) return;
  int n = __popcll(m);
  if (s.cnt + n > kCap) {
    s = chunk_refresh(b, s, k, kSlack);
    s.cnt = uni(s.cnt);
    s.thr = uni(s.thr);
    s.ovf = uni(s.ovf);
    if (s.ovf) return;
    ins = valid && key >= s.thr;
    m = __ballot(ins);
    n = __popcll(m);
  }
  if (ins) {
    const int p = s.cnt + mbcnt(m);
    b->key[p] = key;
    b->base[p] = base;
    raw_put(&b->val[p], raw);
  }
  s.cnt += n;
}

// ------------------------------------------------------------------------------------------
// radix select over a row in global memory (filters the chunk buffers do not serve)
// ------------------------------------------------------------------------------------------

struct SelectOut {
  uint32_t key;   // selected key
  bool reached;   // false: the total weight above lo stays below the target
};

// Largest key t >= lo with W(t) = sum{w(x) : key(x) >= t} >= target, keys
// below lo excluded.  kw(x, key, w) reads token x.  Block-wide.
template <class KW>
__device__ SelectOut block_select(KW kw, int V, uint32_t lo, double target, int key_bits, double* hist,
                                  double* s_d, uint32_t* s_u) {
  const int tid = threadIdx.x, lane = lane_id();
  uint32_t prefix = 0;
  double above = 0.0;
  SelectOut out;
  out.reached = true;
  for (int shift = 24; shift >= 32 - key_bits; shift -= 8) {
    for (int b = tid; b < 256; b += kBlock) hist[b] = 0.0;
    __syncthreads();
    const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
    for (int x = tid; x < V; x += kBlock) {
      uint32_t key;
      double w;
      kw(x, key, w);
      if (key >= lo && (key & hmask) == prefix && w != 0.0) atomicAdd(&hist[(key >> shift) & 255u], w);
    }
    __syncthreads();
    if (tid < 64) {
      double h0 = hist[lane * 4], h1 = hist[lane * 4 + 1], h2 = hist[lane * 4 + 2], h3 = hist[lane * 4 + 3];
      double local = (h0 + h1) + (h2 + h3), suf = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        double t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
      }
      const uint64_t okm = __ballot(above + suf >= target);
      if (okm == 0ull) {
        if (lane == 0) s_u[1] = 1u;  // not reached
      } else {
        const int L = 63 - __clzll((long long)okm);
        double cum = __shfl(above + suf - local, L);
        const double b3 = __shfl(h3, L), b2 = __shfl(h2, L), b1 = __shfl(h1, L);
        int d;
        if (cum + b3 >= target) {
          d = 3;
        } else {
          cum += b3;
          if (cum + b2 >= target) {
            d = 2;
          } else {
            cum += b2;
            if (cum + b1 >= target) {
              d = 1;
            } else {
              cum += b1;
              d = 0;
            }
          }
        }
        if (lane == 0) {
          s_u[0] = (uint32_t)(L * 4 + d);
          s_u[1] = 0u;
          s_d[0] = cum;
        }
      }
    }
    __syncthreads();
    if (s_u[1]) {
      out.reached = false;
      out.key = lo;
      __syncthreads();
      return out;
    }
    prefix |= s_u[0] << shift;
    above = s_d[0];
    __syncthreads();
  }
  out.key = prefix;
  return out;
}

// sum of w(x) over key(x) >= lo
template <class KW>
__device__ double block_sum_above(KW kw, int V, uint32_t lo, double* red) {
  double s = 0.0;
  for (int x = threadIdx.x; x < V; x += kBlock) {
    uint32_t key;
    double w;
    kw(x, key, w);
    if (key >= lo) s += w;
  }
  return block_sum_d(s, red);
}

// ------------------------------------------------------------------------------------------
// shared memory
// ------------------------------------------------------------------------------------------

// Result of one distribution's top-k / top-p filter.
struct MergeOut {
  double mass;      // kept mass (target: sum of 2^((l - m) * c); draft: sum of q^(1/T))
  float cut;        // keep iff value >= cut
  uint32_t cutkey;  // the same as an order key
  int nk;           // top-k tokens left at the front of the key / id / weight arrays
  int ok;           // 0: the buffers cannot decide (ties); the radix select does
};

template <class LT>
struct RowShared {
  // target and draft chunk buffers; once the gather has read them they hold
  // the fp64 weights of the tie path and the radix-select histogram
  ChunkBuf<typename LT::Raw> pb[kWaves];
  ChunkBuf<F32::Raw> qb[kWaves];
  alignas(16) uint32_t skey[2][kWaves * kSeg];   // gathered tokens, one segment per wave
  alignas(16) int sid[2][kWaves * kSeg];
  int scnt[2][kWaves];
  ChunkState ps[kWaves], qs[kWaves];
  float xm[kWaves];
  uint32_t xqb[kWaves];
  uint32_t xlb[kWaves];
  double xr[kWaves];
  double xz[kWaves];
  MergeOut mo[2];
  double red_d[kWaves];
  float red_f[kWaves];
  uint32_t red_u[kWaves];
  int red_i[kWaves];
  double sel_d[2];
  uint32_t sel_u[2];
};


// ------------------------------------------------------------------------------------------
// banned tokens: a request's ascending list in LDS; a banned token reads as a
// -inf logit and a zero draft probability wherever a row is read
// ------------------------------------------------------------------------------------------

// Walks the list along consecutive 512-token wave ranges: ban_mask(lo) gives
// this lane the mask of its 8 tokens lo + 8 * lane .. + 7 and consumes the ids
// below lo + 512, 64 at a time (the list is ascending, so those ids are a
// prefix of the 64 read).  Wave-uniform state.
struct BanWalk {
  int ptr, n;
};
__device__ inline BanWalk ban_start(const LDS_AS int* ban, int n) {
  BanWalk b;
  b.ptr = 0;
  b.n = uni(n);
  return b;
}
__device__ inline uint32_t ban_mask(BanWalk& b, const LDS_AS int* ban, int lo) {
  uint32_t m = 0u;
  const int lane = lane_id();
  while (b.ptr < b.n) {
    const int id = b.ptr + lane < b.n ? ban[b.ptr + lane] : INT_MAX;
    const uint64_t below = __ballot(id < lo + 512);
    uint64_t in = __ballot(id >= lo && id < lo + 512);
    while (in) {
      const int t = __builtin_amdgcn_readlane(id, __ffsll((unsigned long long)in) - 1) - lo;
      if ((t >> 3) == lane) m |= 1u << (t & 7);
      in &= in - 1;
    }
    const int c = __popcll(below);
    b.ptr += c;
    if (c < 64) break;
  }
  return m;
}
__device__ inline bool ban_has(const LDS_AS int* ban, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ban[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo < n && ban[lo] == x;
}
// masked tokens of one lane's raw step: -inf logits, zero probabilities
__device__ inline void ban_apply(Bf16::Raw& r, uint32_t m) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if ((m >> t) & 1u) {
      const uint32_t w = r.a[t >> 1];
      r.a[t >> 1] = (t & 1) ? ((w & 0x0000ffffu) | 0xff800000u) : ((w & 0xffff0000u) | 0x0000ff80u);
    }
}
__device__ inline void ban_apply(F32::Raw& r, uint32_t m, uint32_t fill) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if ((m >> t) & 1u) r.a[t] = fill;
    if ((m >> (t + 4)) & 1u) r.b[t] = fill;
  }
}
__device__ inline void ban_logits(Bf16::Raw& r, uint32_t m) { ban_apply(r, m); }
__device__ inline void ban_logits(F32::Raw& r, uint32_t m) { ban_apply(r, m, 0xff800000u); }

// ------------------------------------------------------------------------------------------
// repetition penalties: a row's ascending list in LDS with each token's
// additive delta d.  A listed logit l reads as (l > 0 ? l / theta : l * theta)
// - d, in float32 and rounded to the logits' type; a listed draft probability
// q reads as q * exp(-d) (in double, then float), the same shift on the
// probability scale.  A banned token still reads as -inf / 0.
// ------------------------------------------------------------------------------------------

// A row's token lists (wave-uniform).
struct Toks {
  const LDS_AS int* ban;    // banned tokens, ascending
  int nban;
  const LDS_AS int* pid;    // penalised tokens, ascending
  const LDS_AS float* pd;   // their deltas
  LDS_AS float* stage;      // this wave's 512 staging slots (NaN when empty)
  int npen;
  float theta;              // repetition penalty
};

__device__ inline float pen_logit(float l, float theta, float d) {
#pragma clang fp contract(off)
  const float l1 = l > 0.f ? l / theta : l * theta;
  return l1 - d;
}
// float32 to bf16 bits, to nearest even; NaN stays NaN
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ inline float pen_value(Bf16*, float l, float theta, float d) {
  return __uint_as_float(bf16_rne(pen_logit(l, theta, d)) << 16);
}
__device__ inline float pen_value(F32*, float l, float theta, float d) { return pen_logit(l, theta, d); }
__device__ inline float pen_prob(float q, float d) { return (float)((double)q * exp(-(double)d)); }

// Rewrites the listed tokens of one lane's raw step; d[e] is token e's delta
// or NaN (not listed).
__device__ inline void pen_apply(Bf16::Raw& r, const float d[8], float theta) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (d[e] == d[e]) {
      const uint32_t w = r.a[e >> 1];
      const uint32_t bits = (e & 1) ? (w >> 16) : (w & 0xffffu);
      const uint32_t nb = bf16_rne(pen_logit(__uint_as_float(bits << 16), theta, d[e]));
      r.a[e >> 1] = (e & 1) ? ((w & 0x0000ffffu) | (nb << 16)) : ((w & 0xffff0000u) | nb);
    }
}
__device__ inline void pen_apply(F32::Raw& r, const float d[8], float theta) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (d[e] == d[e]) {
      if (e < 4) r.a[e] = __float_as_uint(pen_logit(__uint_as_float(r.a[e]), theta, d[e]));
      else r.b[e - 4] = __float_as_uint(pen_logit(__uint_as_float(r.b[e - 4]), theta, d[e]));
    }
}
__device__ inline void pen_apply_q(F32::Raw& r, const float d[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (d[e] == d[e]) {
      if (e < 4) r.a[e] = __float_as_uint(pen_prob(__uint_as_float(r.a[e]), d[e]));
      else r.b[e - 4] = __float_as_uint(pen_prob(__uint_as_float(r.b[e - 4]), d[e]));
    }
}

// Walks the penalty list along consecutive 512-token wave ranges as ban_mask
// walks the ban list.  The ids of the range [lo, lo + 512) write their deltas
// into the wave's staging slots (ids are distinct, so no two lanes share a
// slot); each lane then reads the 8 slots of its tokens lo + 8 * lane .. + 7,
// rewrites the listed ones (and their draft probabilities when q_on), and
// resets those slots to NaN.  The cost per step does not grow with the number
// of listed tokens in it.
struct PenWalk {
  int ptr, n;
};
__device__ inline PenWalk pen_start(int n) {
  PenWalk b;
  b.ptr = 0;
  b.n = uni(n);
  return b;
}
template <class LR>
__device__ inline void pen_walk(PenWalk& b, const Toks& tk, int lo, LR& l, F32::Raw& q, bool q_on) {
  const int lane = lane_id();
  uint64_t wrote = 0ull;
  while (b.ptr < b.n) {
    const bool ok = b.ptr + lane < b.n;
    const int id = ok ? tk.pid[b.ptr + lane] : INT_MAX;
    const float d = ok ? tk.pd[b.ptr + lane] : 0.f;
    const bool inr = id >= lo && id < lo + 512;
    if (inr) tk.stage[id - lo] = d;
    wrote |= __ballot(inr);
    const int c = __popcll(__ballot(id < lo + 512));
    b.ptr += c;
    if (c < 64) break;
  }
  if (!wrote) return;
  wave_lds_sync();
  float dv[8];
  {
    const LDS_AS f32x4* sp = reinterpret_cast<const LDS_AS f32x4*>(tk.stage + lane * kCh);
    const f32x4 x = sp[0], y = sp[1];
    dv[0] = x.x; dv[1] = x.y; dv[2] = x.z; dv[3] = x.w;
    dv[4] = y.x; dv[5] = y.y; dv[6] = y.z; dv[7] = y.w;
  }
  bool hit = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) hit |= dv[e] == dv[e];
  if (hit) {
    pen_apply(l, dv, tk.theta);
    if (q_on) pen_apply_q(q, dv);
    LDS_AS f32x4* sp = reinterpret_cast<LDS_AS f32x4*>(tk.stage + lane * kCh);
    const float nan = __uint_as_float(0x7fffffffu);
    sp[0] = f32x4{nan, nan, nan, nan};
    sp[1] = f32x4{nan, nan, nan, nan};
  }
  wave_lds_sync();
}

// index of x in an ascending list, or -1
__device__ inline int tok_find(const LDS_AS int* ids, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ids[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return (lo < n && ids[lo] == x) ? lo : -1;
}
// token x's logit l / draft probability q as the row's lists make it
template <class LT>
__device__ inline float tok_logit(const Toks& tk, int x, float l) {
  if (tk.npen) {
    const int k = tok_find(tk.pid, tk.npen, x);
    if (k >= 0) l = pen_value((LT*)nullptr, l, tk.theta, tk.pd[k]);
  }
  if (tk.nban && ban_has(tk.ban, tk.nban, x)) l = -INFINITY;
  return l;
}
__device__ inline float tok_prob(const Toks& tk, int x, float q) {
  if (tk.npen) {
    const int k = tok_find(tk.pid, tk.npen, x);
    if (k >= 0) q = pen_prob(q, tk.pd[k]);
  }
  if (tk.nban && ban_has(tk.ban, tk.nban, x)) q = 0.f;
  return q;
}
__device__ inline Toks toks(const LDS_AS int* ban, int nban, const LDS_AS int* pid, const LDS_AS float* pd,
                            LDS_AS float* stage, int npen, float theta) {
  Toks t;
  t.ban = ban;
  t.nban = uni(nban);
  t.pid = pid;
  t.pd = pd;
  t.stage = stage;
  t.npen = uni(npen);
  t.theta = uni(theta);
  return t;
}

// ------------------------------------------------------------------------------------------
// kept set from the candidate buffers (one wave per distribution)
// ------------------------------------------------------------------------------------------

// Sums over u < n (n a multiple of 8, at most 64) of e[u] where keys[u] >= key
// (ids[u] <= id for the draw), read from LDS with broadcast vector loads and
// accumulated in eight independent partial sums; unused slots hold key 0 (id
// INT_MAX) and weight 0.
__device__ inline double tree8(const double p[8]) {
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}
// Eight weights of one group, loaded unconditionally (an empty asm pins the
// loads, which the compiler would otherwise turn into masked per-lane loads
// under the select).
__device__ inline void lds_load8_f64(const LDS_AS double* e, double ev[8]) {
  typedef double f64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    f64x2 x = *(const LDS_AS f64x2*)(e + 2 * h);
    asm volatile("" : "+v"(x));
    ev[2 * h] = x.x;
    ev[2 * h + 1] = x.y;
  }
}
__device__ inline double lds_sum_key_ge(const LDS_AS uint32_t* keys, const LDS_AS double* e, int n, uint32_t key) {
  double part[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) part[t] = 0.0;
  for (int u = 0; u < n; u += 8) {
    const u32x4 k0 = *(const LDS_AS u32x4*)(keys + u);
    const u32x4 k1 = *(const LDS_AS u32x4*)(keys + u + 4);
    double ev[8];
    lds_load8_f64(e + u, ev);
    const uint32_t kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) part[t] += (kv[t] >= key) ? ev[t] : 0.0;
  }
  return tree8(part);
}
__device__ inline double lds_sum_id_le(const LDS_AS int* ids, const LDS_AS double* w, int n, int id) {
  double part[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) part[t] = 0.0;
  for (int u = 0; u < n; u += 8) {
    const u32x4 i0 = *(const LDS_AS u32x4*)(ids + u);
    const u32x4 i1 = *(const LDS_AS u32x4*)(ids + u + 4);
    double wv[8];
    lds_load8_f64(w + u, wv);
    const int iv[8] = {(int)i0.x, (int)i0.y, (int)i0.z, (int)i0.w, (int)i1.x, (int)i1.y, (int)i1.z, (int)i1.w};
#pragma unroll
    for (int t = 0; t < 8; ++t) part[t] += (iv[t] <= id) ? wv[t] : 0.0;
  }
  return tree8(part);
}

struct MergeIn {
  uint32_t L;         // largest wave threshold: gathered tokens below it are dropped
  int ovf;            // a wave's buffer overflowed
  int k;
  float top_p;
  int pact;
  int draft;          // weights (q / qs)^(1/T) (else 2^((l - m) * c))
  float m, T, qinv;
  double cd;          // log2(e) / T in fp64 (target weights)
};

__device__ inline double merge_weight(const MergeIn& in, float v) {
  return in.draft ? temper_q(v, in.T, in.qinv) : exp2(((double)v - (double)in.m) * in.cd);
}

__device__ inline void unpack_raw(const Bf16::Raw& r, float v[8]) { Bf16::unpack(r, v); }
__device__ inline void unpack_raw(const F32::Raw& r, float v[8]) { F32::unpack(r, v); }

// One wave copies the tokens of its own buffered chunks whose key reaches L
// (tokens past the row end excluded) into its segment; returns their count
// (more than kSeg: the segment overflowed).
template <class R>
__device__ inline int gather_tokens(const LDS_AS ChunkBuf<R>* b, int cnt, uint32_t L, int V, LDS_AS uint32_t* skey,
                                    LDS_AS int* sid) {
  const int lane = lane_id();
  cnt = uni(cnt);
  L = uni(L);
  int n = 0;
  for (int e0 = 0; e0 < cnt; e0 += 64) {
    const int e = e0 + lane;
    const bool h = e < cnt && b->key[e] >= L;
    float v[8];
    int base = 0;
    if (h) {
      R raw;
      raw_get(&b->val[e], raw);
      unpack_raw(raw, v);
      base = b->base[e];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t key = h ? okey(v[t]) : 0u;
      const bool take = h && base + t < V && key >= L;
      const uint64_t mb = __ballot(take);
      const int p = n + mbcnt(mb);
      if (take && p < kSeg) {
        skey[p] = key;
        sid[p] = base + t;
      }
      n += __popcll(mb);
    }
  }
  return n;
}

// The gathered segments hold every token of the row whose key reaches L = the
// largest wave threshold, a lower bound of the row's k-th largest key, so the
// exact k-th largest key K is found among them by bisection (below the common
// prefix of their smallest and largest key; bf16 keys end in 16 equal bits).
// The tokens at or above K are weighed in fp64 and top-p keeps the smallest
// run of whole tie groups, largest values first, whose mass reaches top_p of
// the top-k mass.  Run by a single wave.  On return the top-k tokens are at
// the front of skey / sid (nk of them) with their fp64 weights in mmass.
template <bool BF16KEYS>
__device__ __noinline__ MergeOut wave_merge(MergeIn in, LDS_AS uint32_t* skey, LDS_AS int* sid, const LDS_AS int* scnt,
                                            LDS_AS double* mmass) {
  const int lane = lane_id();
  in.L = uni(in.L);
  in.ovf = uni(in.ovf);
  in.k = uni(in.k);
  in.pact = uni(in.pact);
  in.draft = uni(in.draft);
  in.top_p = uni(in.top_p);
  in.m = uni(in.m);
  in.qinv = uni(in.qinv);
  in.cd = uni(in.cd);
  in.T = uni(in.T);
  MergeOut out;
  out.ok = 0;
  out.nk = 0;
  out.cut = -INFINITY;
  out.cutkey = 0u;
  out.mass = 0.0;
  if (in.ovf) return out;
  int segn[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    segn[w] = uni(scnt[w]);
    if (segn[w] > kSeg) return out;
  }
  constexpr int G = kSeg / 64;
  uint32_t kk[kWaves * G];
  int ii[kWaves * G];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int e = 64 * g + lane;
      bool h = e < segn[w];
      kk[w * G + g] = h ? skey[w * kSeg + e] : 0u;
      if (kk[w * G + g] < in.L) {
        kk[w * G + g] = 0u;
        h = false;
      }
      ii[w * G + g] = h ? sid[w * kSeg + e] : 0;
      if (h) {
        kmax = max(kmax, kk[w * G + g]);
        kmin = min(kmin, kk[w * G + g]);
      }
    }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  // unused slots hold key 0 and every probe T is >= 1: no guards, and the
  // group counts are independent (summed as a tree)
  auto count_ge = [&](uint32_t T) {
    int c[kWaves * G];
#pragma unroll
    for (int t = 0; t < kWaves * G; ++t) c[t] = __popcll(__ballot(kk[t] >= T));
#pragma unroll
    for (int h = 1; h < kWaves * G; h <<= 1)
#pragma unroll
      for (int t = 0; t + h < kWaves * G; t += 2 * h) c[t] += c[t + h];
    return c[0];
  };
  // The top-k set is {key >= K} for the k-th largest key K (ties included).
  // K is decided 8 bits at a time below the common prefix of the gathered
  // keys: an LDS histogram of the next digit over the keys that share the
  // decided prefix, then the largest digit whose keys, with all larger ones,
  // number at least k.  Once exactly k keys reach the decided prefix they are
  // the top-k set, and K is replaced by their smallest key below.
  uint32_t K = kmin;
  if (kmin != kmax) {
    LDS_AS int* hist = (LDS_AS int*)mmass;  // 256 bins; the weights come later
    const int top = 31 - __clz((int)(kmin ^ kmax));
    uint32_t P = kmin & ~((2u << top) - 1u);
    int above = 0;  // keys whose decided bits exceed P's
    int hi = top;
    constexpr int lo = BF16KEYS ? 16 : 0;  // bf16 keys end in 16 equal bits
    bool exact = false;
    while (hi >= lo) {
      const int d = min(8, hi - lo + 1);
      const int sh = hi - d + 1;
      const uint32_t dmask = (1u << d) - 1u;
      *(LDS_AS u32x4*)(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < kWaves * G; ++t) {
        const uint32_t x = kk[t];
        const bool match = x != 0u && (hi == 31 || ((x ^ P) >> (hi + 1)) == 0u);
        if (match) __hip_atomic_fetch_add(hist + ((x >> sh) & dmask), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      wave_lds_sync();
      const u32x4 b = *(const LDS_AS u32x4*)(hist + 4 * lane);
      const int S = wave_incl_scan_i32((int)(b.x + b.y + b.z + b.w));
      const int T = __builtin_amdgcn_readlane(S, 63);
      // keys with digit >= 4 * lane + i
      const int s3 = T - S + (int)b.w, s2 = s3 + (int)b.z, s1 = s2 + (int)b.y, s0 = s1 + (int)b.x;
      const int Ls = 63 - __clzll((long long)__ballot(above + s0 >= in.k));  // lane 0 always qualifies
      const int pick = (above + s3 >= in.k) ? 3 : (above + s2 >= in.k) ? 2 : (above + s1 >= in.k) ? 1 : 0;
      const int sp = pick == 3 ? s3 : pick == 2 ? s2 : pick == 1 ? s1 : s0;
      const int bp = (int)(pick == 3 ? b.w : pick == 2 ? b.z : pick == 1 ? b.y : b.x);
      const int D = 4 * Ls + __builtin_amdgcn_readlane(pick, Ls);
      const int cge = above + __builtin_amdgcn_readlane(sp, Ls);  // keys >= the new prefix
      P |= (uint32_t)D << sh;
      above = cge - __builtin_amdgcn_readlane(bp, Ls);
      hi = sh - 1;
      wave_lds_sync();
      if (cge == in.k) {
        exact = true;
        break;
      }
    }
    if (BF16KEYS && !exact && count_ge(P | 0xffffu) >= in.k) P |= 0xffffu;
    K = P;
  }
  {
    uint32_t kmin2 = 0xffffffffu;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (64 * g + lane < segn[w] && kk[w * G + g] >= K) kmin2 = min(kmin2, kk[w * G + g]);
    K = wave_min_u32(kmin2);
  }
  // the top-k set, compacted to the front of the segment area
  wave_lds_sync();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (64 * g < segn[w]) {
        const bool take = 64 * g + lane < segn[w] && kk[w * G + g] >= K;
        const uint64_t mb = __ballot(take);
        if (take) {
          skey[nk + mbcnt(mb)] = kk[w * G + g];
          sid[nk + mbcnt(mb)] = ii[w * G + g];
        }
        nk += __popcll(mb);
      }
    }
  wave_lds_sync();
  uint32_t cutkey = K;
  if (nk <= 64) {
    // one entry per lane
    const bool h = lane < nk;
    const uint32_t key = h ? skey[lane] : 0u;
    const int id = h ? sid[lane] : INT_MAX;
    const double e = h ? merge_weight(in, okey_value(key)) : 0.0;
    // the 64 slots padded (key 0, id INT_MAX, weight 0) for the LDS sums here
    // and in the draw
    wave_lds_sync();
    skey[lane] = key;
    sid[lane] = id;
    mmass[lane] = e;
    wave_lds_sync();
    const double zk = wave_sum_f64(e);
    double mass = zk;
    if (in.pact) {
      // cum = mass of the entries whose key is >= this lane's key
      const double cum = lds_sum_key_ge(skey, mmass, (nk + 7) & ~7, key);
      const double target = (double)in.top_p * zk;
      const uint32_t best = wave_max_u32((h && cum >= target) ? key : 0u);
      if (best != 0u) {  // else rounding kept the run below target: keep the whole top-k set
        cutkey = best;
        const uint64_t at = __ballot(h && key == best);
        mass = readlane_d(cum, __ffsll((unsigned long long)at) - 1);
      }
    }
    out.mass = mass;
  } else {
    // many values tied at the k-th largest: weights in LDS, quadratic top-p
    double zp = 0.0;
    for (int t = lane; t < nk; t += 64) {
      const double e = merge_weight(in, okey_value(skey[t]));
      mmass[t] = e;
      zp += e;
    }
    const double zk = wave_sum_d(zp);
    wave_lds_sync();
    if (in.pact) {
      const double target = (double)in.top_p * zk;
      uint32_t best = 0u;
      for (int t = lane; t < nk; t += 64) {
        const uint32_t kt = skey[t];
        double cum = 0.0;
        for (int u = 0; u < nk; ++u) cum += (skey[u] >= kt) ? mmass[u] : 0.0;
        if (cum >= target) best = max(best, kt);
      }
      best = wave_max_u32(best);
      if (best != 0u) cutkey = best;
    }
    double zc = 0.0;
    for (int t = lane; t < nk; t += 64)
      if (skey[t] >= cutkey) zc += mmass[t];
    out.mass = wave_sum_d(zc);
  }
  out.cut = okey_value(cutkey);
  out.cutkey = cutkey;
  out.nk = nk;
  out.ok = 1;
  return out;
}

// ------------------------------------------------------------------------------------------
// the draw from a row's kept list (rows with top-k)
// ------------------------------------------------------------------------------------------

struct DrawIn {
  int nk;             // top-k tokens at the front of the key / id / weight arrays
  uint32_t cutkey;    // a token is kept iff its key >= cutkey
  double zk;          // kept target mass
  int mode;           // 0: p'; 1: max(0, p' - q'); 2: p' with the draft token removed
  const float* qrow;  // mode 1: the draft row
  float cut_q, T;     // mode 1: draft cut and temperature
  float qinv;         // mode 1: 1 / qs
  double rk;          // mode 1: kept draft mass
  int y;              // mode 2: the draft token
  float us;           // the request's draw uniform
};

struct DrawOut {
  double s;           // mass S of the weights drawn from
  int z;              // drawn token
  int pad;
};

// Weights w over the kept tokens (every token with p' > 0 is among them, so
// w is zero elsewhere); if they sum to zero, w = p'.  z = the smallest id
// whose running sum of w in ascending id exceeds u * S, else the largest id
// with w > 0.  Run by a single wave; wbuf is LDS scratch for more than 64
// kept tokens.
__device__ __noinline__ DrawOut wave_draw(DrawIn in, const LDS_AS uint32_t* skey, const LDS_AS int* sid,
                                          const LDS_AS double* ke, LDS_AS double* wbuf, const LDS_AS int* ban,
                                          int nban, const LDS_AS int* pid, const LDS_AS float* pd, int npen) {
  const int lane = lane_id();
  in.nk = uni(in.nk);
  in.cutkey = uni(in.cutkey);
  in.zk = uni(in.zk);
  in.mode = uni(in.mode);
  in.qrow = uni(in.qrow);
  in.cut_q = uni(in.cut_q);
  in.T = uni(in.T);
  in.qinv = uni(in.qinv);
  in.rk = uni(in.rk);
  in.y = uni(in.y);
  in.us = uni(in.us);
  const Toks tk = toks(ban, nban, pid, pd, nullptr, npen, 1.f);
  auto weight = [&](bool keep, int id, double e, double& p) {
    p = keep ? e / in.zk : 0.0;
    double w = p;
    if (in.mode == 1) {
      double q = 0.0;
      if (keep) {
        const float qx = tok_prob(tk, id, F32::at(in.qrow, (size_t)id));
        q = (qx >= in.cut_q) ? temper_q(qx, in.T, in.qinv) / in.rk : 0.0;
      }
      w = p - q > 0.0 ? p - q : 0.0;
    } else if (in.mode == 2) {
      w = (id == in.y) ? 0.0 : p;
    }
    return w;
  };
  DrawOut out;
  out.pad = 0;
  uint32_t best = 0xffffffffu, last = 0u;  // last: largest id with w > 0, plus one
  if (in.nk <= 64) {
    const bool h = lane < in.nk;
    const bool keep = h && skey[lane] >= in.cutkey;
    const int id = sid[lane];
    double p;
    double w = weight(keep, id, h ? ke[lane] : 0.0, p);
    double S = wave_sum_f64(w);
    if (S == 0.0) {
      w = p;
      S = wave_sum_f64(p);
    }
    const double tau = (double)in.us * S;
    // running sum at this lane's id (the 64 id slots are padded with INT_MAX)
    wbuf[lane] = w;
    wave_lds_sync();
    const double cum = lds_sum_id_le(sid, wbuf, (in.nk + 7) & ~7, id);
    if (w > 0.0) {
      if (cum > tau) best = (uint32_t)id;
      last = (uint32_t)id + 1u;
    }
    out.s = S;
  } else {
    // many tokens tied at the k-th largest value: weights in LDS, quadratic sums
    double sp = 0.0, sw = 0.0;
    for (int t = lane; t < in.nk; t += 64) {
      double p;
      const double w = weight(skey[t] >= in.cutkey, sid[t], ke[t], p);
      wbuf[t] = w;
      sw += w;
      sp += p;
    }
    double S = wave_sum_d(sw);
    wave_lds_sync();
    if (S == 0.0) {
      for (int t = lane; t < in.nk; t += 64) wbuf[t] = skey[t] >= in.cutkey ? ke[t] / in.zk : 0.0;
      S = wave_sum_d(sp);
      wave_lds_sync();
    }
    const double tau = (double)in.us * S;
    for (int t = lane; t < in.nk; t += 64) {
      if (!(wbuf[t] > 0.0)) continue;
      const int id = sid[t];
      double cum = 0.0;
      for (int u = 0; u < in.nk; ++u) cum += (sid[u] <= id) ? wbuf[u] : 0.0;
      if (cum > tau) best = min(best, (uint32_t)id);
      last = max(last, (uint32_t)id + 1u);
    }
    out.s = S;
  }
  best = wave_min_u32(best);
  last = wave_max_u32(last);
  out.z = best != 0xffffffffu ? (int)best : (int)last - 1;
  return out;
}

// A row of target logits (bf16 or fp32) or draft probabilities (fp32).
struct RowRef {
  const void* row;
  int V;
  bool bf16;
};

__device__ inline float row_value(const RowRef& r, int x) {
  return r.bf16 ? Bf16::at(reinterpret_cast<const uint16_t*>(r.row), (size_t)x)
                : F32::at(reinterpret_cast<const float*>(r.row), (size_t)x);
}

// Filters the candidate buffers do not serve: radix selects that re-read the row.
// Returns the cut value (-inf: keep all) and the kept mass in *mass.
struct GeneralArgs {
  const void* row;
  int V;
  bool bf16, draft;
  float m;
  float T;        // temperature
  float qinv;     // draft rows: 1 / qs
  bool temper;
  int k;
  bool kact;
  float top_p;
  bool pact;
  double total;   // unfiltered mass of the row
};

struct Filtered {
  float cut;
  double mass;
};

__device__ __noinline__ Filtered general_filter(GeneralArgs g, LDS_AS double* hist, LDS_AS double* sel_d,
                                                LDS_AS uint32_t* sel_u, LDS_AS double* red, const LDS_AS int* ban,
                                                int nban, const LDS_AS int* pid, const LDS_AS float* pd, int npen,
                                                float theta) {
  g.row = uni(g.row);
  g.V = uni(g.V);
  g.bf16 = uni((int)g.bf16);
  g.draft = uni((int)g.draft);
  g.m = uni(g.m);
  g.T = uni(g.T);
  g.qinv = uni(g.qinv);
  g.temper = uni((int)g.temper);
  const Scale2 c = uni_s2(target_scale(g.T));
  const DraftW dw = uni_dw(draft_w(g.T));
  g.k = uni(g.k);
  g.kact = uni((int)g.kact);
  g.top_p = uni(g.top_p);
  g.pact = uni((int)g.pact);
  g.total = uni(g.total);
  const Toks tk = toks(ban, nban, pid, pd, nullptr, npen, theta);
  RowRef ka;
  ka.row = g.row;
  ka.V = g.V;
  ka.bf16 = g.bf16;
  auto weight = [&](float v) -> double {
    return g.draft ? (g.temper ? temper_w64(v, dw, g.qinv) : (double)v) : (double)mass_p32(v, g.m, c);
  };
  auto value = [&](int x) -> float {
    const float v = row_value(ka, x);
    if (!tk.nban && !tk.npen) return v;
    return g.draft ? tok_prob(tk, x, v) : (g.bf16 ? tok_logit<Bf16>(tk, x, v) : tok_logit<F32>(tk, x, v));
  };
  auto kw = [&](int x, uint32_t& key, double& w) {
    const float v = value(x);
    key = okey(v);
    w = weight(v);
  };
  auto kc = [&](int x, uint32_t& key, double& w) {
    key = okey(value(x));
    w = 1.0;
  };
  uint32_t lo = 0u;
  if (g.kact)
    lo = block_select(kc, g.V, 0u, (double)g.k, 32, (double*)hist, (double*)sel_d, (uint32_t*)sel_u).key;
  const double zk = g.kact ? block_sum_above(kw, g.V, lo, (double*)red) : g.total;
  uint32_t cutk = lo;
  double zc = zk;
  if (g.pact) {
    SelectOut so = block_select(kw, g.V, lo, (double)g.top_p * zk, 32, (double*)hist, (double*)sel_d,
                                (uint32_t*)sel_u);
    if (so.reached) {
      cutk = so.key;
      zc = block_sum_above(kw, g.V, cutk, (double*)red);
    }
  }
  Filtered f;
  f.cut = (cutk == 0u) ? -INFINITY : okey_value(cutk);
  f.mass = zc;
  return f;
}

// ------------------------------------------------------------------------------------------
// streaming passes
// ------------------------------------------------------------------------------------------

// Stream `nfull` full steps keeping D steps of loads in flight: load(s)
// returns the raw data of step s, proc(raw, s) reduces it.  In the steady
// state every refill is unconditional, so the compiler's wait counters let
// the D - 1 younger loads stay outstanding while the oldest is reduced.
template <int D, class Raw, class Load, class Proc>
__device__ __forceinline__ void ring_stream(int nfull, Load load, Proc proc) {
  Raw ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < nfull) ring[u] = load(u);
  int s0 = 0;
  for (; s0 + 2 * D <= nfull; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const Raw cur = ring[u];
      ring[u] = load(s0 + u + D);
      proc(cur, s0 + u);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const int s = s0 + u;
    if (s < nfull) {
      const Raw cur = ring[u];
      if (s + D < nfull) ring[u] = load(s + D);
      proc(cur, s);
    }
  }
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const int s = s0 + D + u;
    if (s < nfull) proc(ring[u], s);
  }
}

template <class LR>
struct StepRaw {
  LR l;
  F32::Raw q;
};

struct StochState {
  float m;          // running max of this thread's logits
  double z;         // sum of 2^((l - m) * c) over this thread's logits (no top-k)
  double r;         // sum of q at T = 1, else of (q / qs)^(1/T), qs = 2^(scale_e(qbad) - 126) (no top-k)
  float qinv;       // 1 / qs
  uint32_t qbad;    // max raw bits of q (>= 0x7f800000: NaN, inf or sign bit)
  uint32_t lbad;    // max bits of |l| (> 0x7f800000: NaN) (top-k)
  ChunkState ps, qs;
};

// QM: 0 no draft row, 1 draft row at T = 1, 2 draft row at T != 1, 3 draft row at
// 1/T above kPreciseInvT (without top-k: the weights that carry mass in fp64, a
// code path of its own so that the others keep their registers).
template <class LT, bool VEC, int QM, bool CAND, int TOK>
__device__ __forceinline__ void stream_stochastic(const typename LT::T* lrow, const float* qrow, int V, const Scale2& c,
                                                  const DraftW& dw, int k, RowShared<LT>& sh, StochState& st,
                                                  const Toks& tk) {
  typedef typename LT::Raw LR;
  const int tid = threadIdx.x, w = tid >> 6;
  const int nsteps = (V + kStep - 1) / kStep;
  auto process = [&](const LR& lr, const F32::Raw& qr, int base) {
    float v[8];
    LT::unpack(lr, v);
    const float cm = max8(v);
    if (CAND) {
      // with top-k the kept masses come from the candidates alone: only the
      // max and a NaN check are needed from the full row
      st.m = __builtin_fmaxf(st.m, cm);
      uint32_t a[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) a[t] = __float_as_uint(v[t]) & 0x7fffffffu;
      st.lbad = max(st.lbad, max8u(a));
    } else {
      if (cm > st.m) {
        st.z *= (double)mass_p32(st.m, cm, c);
        st.m = cm;
      }
      float e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) e[t] = mass_p32(v[t], st.m, c);
      st.z += (double)(((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
    }
    uint32_t qmax = 0u;
    if (QM) {
      uint32_t u[8];
      F32::bits(qr, u);
      qmax = max8u(u);
      if (QM >= 2 && !CAND && qmax > st.qbad) {
        const int e0 = scale_e(st.qbad), e1 = scale_e(qmax);
        if (e1 > e0) {
          // a q in a higher binade: move the running sum to the new scale
          if (st.r != 0.0) st.r *= scale_step32(e0, e1, dw.invT);
          st.qinv = scale_inv(e1);
        }
      }
      st.qbad = max(st.qbad, qmax);
      if (!CAND) {
        float r[8];
        double hi = 0.0;  // weights formed in fp64 (QM 3)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float qv = __uint_as_float(u[t]);
          if (QM == 1) r[t] = qv;
          else if (QM == 2) r[t] = fast_exp2(smul(fast_log2(qv * st.qinv), dw.invT));
          else r[t] = temper_w32(qv, dw, st.qinv, hi);
        }
        st.r += (double)(((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7])));
        if (QM == 3) st.r += hi;
      }
    }
    if (CAND) {
      const bool valid = base < V;
      chunk_offer((LDS_AS ChunkBuf<LR>*)&sh.pb[w], st.ps, k, valid, okey(cm), base, lr);
      // okey of q >= 0 is its bits with the sign bit set
      if (QM) chunk_offer((LDS_AS ChunkBuf<F32::Raw>*)&sh.qb[w], st.qs, k, valid, qmax | 0x80000000u, base, qr);
    }
  };
  // full steps (every lane's 8 tokens inside the row, vector loads only)
  const int nfull = VEC ? V / kStep : 0;
  const int base0 = tid * kCh;
  BanWalk bw;
  PenWalk pw;
  if (TOK) bw = ban_start(tk.ban, tk.nban);
  if (TOK == 2) pw = pen_start(tk.npen);
  ring_stream<QM ? 5 : 10, StepRaw<LR>>(
      nfull,
      [&](int s) {
        StepRaw<LR> r;
        r.l = LT::load(lrow + base0 + s * kStep);
        if (QM) r.q = F32::load(qrow + base0 + s * kStep);
        return r;
      },
      [&](const StepRaw<LR>& r, int s) {
        if (TOK) {
          StepRaw<LR> b = r;
          if (TOK == 2) pen_walk(pw, tk, s * kStep + w * 512, b.l, b.q, QM != 0);
          const uint32_t m = ban_mask(bw, tk.ban, s * kStep + w * 512);
          if (m) {
            ban_logits(b.l, m);
            if (QM) ban_apply(b.q, m, 0u);
          }
          process(b.l, b.q, base0 + s * kStep);
        } else {
          process(r.l, r.q, base0 + s * kStep);
        }
      });
  int base = base0 + nfull * kStep;
  // the ragged tail (and every step of rows that are not 16-byte aligned)
  for (int s = nfull; s < nsteps; ++s) {
    LR lr = load_logits<LT, VEC>(lrow, base, V);
    F32::Raw qr{};
    if (QM) qr = load_probs<VEC>(qrow, base, V);
    if (TOK == 2) pen_walk(pw, tk, s * kStep + w * 512, lr, qr, QM != 0);
    if (TOK) {
      const uint32_t m = ban_mask(bw, tk.ban, s * kStep + w * 512);
      if (m) {
        ban_logits(lr, m);
        if (QM) ban_apply(qr, m, 0u);
      }
    }
    process(lr, qr, base);
    base += kStep;
  }
}

// Greedy rows: argmax (lowest id among equal maxima) and a running sum that
// flags NaN / +inf for an exact re-check.
template <class LT, bool VEC, int TOK>
__device__ __forceinline__ void stream_greedy(const typename LT::T* lrow, int V, float& best, int& bidx, float& acc,
                                              const Toks& tk) {
  typedef typename LT::Raw LR;
  const int tid = threadIdx.x, w = tid >> 6;
  const int nsteps = (V + kStep - 1) / kStep;
  // m: banned tokens of the step (read as -inf, left out of the running sum)
  auto process = [&](const LR& lr, int base, uint32_t m) {
    float v[8];
    LT::unpack(lr, v);
    if (base < V) {
      float a[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) a[t] = ((m >> t) & 1u) ? 0.f : v[t];
      acc += ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
      const float cm = max8(v);
      if (cm > best) {
        int f = 7;
#pragma unroll
        for (int t = 7; t >= 0; --t)
          if (v[t] == cm) f = t;
        best = cm;
        bidx = base + f;
      }
    }
  };
  const int nfull = VEC ? V / kStep : 0;
  const int base0 = tid * kCh;
  BanWalk bw;
  PenWalk pw;
  if (TOK) bw = ban_start(tk.ban, tk.nban);
  if (TOK == 2) pw = pen_start(tk.npen);
  auto masked = [&](const LR& r, int s, int base) {
    if (TOK) {
      LR b = r;
      if (TOK == 2) {
        F32::Raw none;
        pen_walk(pw, tk, s * kStep + w * 512, b, none, false);
      }
      const uint32_t m = ban_mask(bw, tk.ban, s * kStep + w * 512);
      if (m) ban_logits(b, m);
      process(b, base, m);
    } else {
      process(r, base, 0u);
    }
  };
  ring_stream<8, LR>(
      nfull, [&](int s) { return LT::load(lrow + base0 + s * kStep); },
      [&](const LR& r, int s) { masked(r, s, base0 + s * kStep); });
  int base = base0 + nfull * kStep;
  for (int s = nfull; s < nsteps; ++s) {
    masked(load_logits<LT, VEC>(lrow, base, V), s, base);
    base += kStep;
  }
}

// ------------------------------------------------------------------------------------------
// row processing
// ------------------------------------------------------------------------------------------

template <class LT, bool VEC, int TOK>
__device__ __forceinline__ void greedy_row(const Args& a, const Req& rq, int i, int j, RowShared<LT>& sh,
                                           const Toks& tk) {
  typedef typename LT::T ET;
  const int G = a.G, V = a.V, tid = threadIdx.x;
  const size_t row = (size_t)i * (G + 1) + j;  // the row record
  const ET* lrow = reinterpret_cast<const ET*>(a.logits) + (size_t)rq.trow * (size_t)V;
  float best = -INFINITY, acc = 0.f;
  int bidx = -1;
  stream_greedy<LT, VEC, TOK>(lrow, V, best, bidx, acc, tk);
  __builtin_amdgcn_s_setprio(2);
  const float gbest = block_max_f(best, sh.red_f);
  int cand = (best == gbest && bidx >= 0) ? bidx : INT_MAX;
  cand = block_min_i(cand, sh.red_i);
  // the running sum is finite unless the row holds NaN, an infinity, or
  // values whose sum overflows: then look exactly for NaN / +inf
  const int suspicious = block_max_i(isfinite(acc) ? 0 : 1, sh.red_i);
  int bad = 0;
  if (suspicious) {
    for (int x = tid; x < V; x += kBlock) {
      float l = LT::at(lrow, (size_t)x);
      if (TOK) l = tok_logit<LT>(tk, x, l);
      bad |= (l != l) || (l == INFINITY);
    }
    bad = block_max_i(bad, sh.red_i);
  }
  if (tid == 0) {
    const int fault = (bad || gbest == INFINITY || cand == INT_MAX) ? kFaultTargetRow : 0;
    const int y = j < rq.gamma ? a.ids[(size_t)rq.id0 + j] : -1;
    RowStats s;
    s.m = gbest;
    s.cut_p = -INFINITY;
    s.cut_q = -INFINITY;
    s.argmax = cand == INT_MAX ? -1 : cand;
    s.z = 0.0;
    s.r = 0.0;
    s.p_y = NAN;
    s.q_y = NAN;
    s.s = NAN;
    s.flags = ((!a.synthetic && j < rq.gamma && y == cand) ? 1 : 0) | (fault << 8);
    s.draw = s.argmax;  // a greedy row's token is its argmax
    publish(a.stats + row, s);
    note_row(a, i, j, s.flags & 1, fault, false);
  }
}

template <class LT, bool VEC, int TOK>
__device__ __forceinline__ void stochastic_row(const Args& a, const Req& rq, int i, int j, RowShared<LT>& sh,
                                               const Toks& tk) {
  typedef typename LT::T ET;
  const int G = a.G, V = a.V;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const size_t row = (size_t)i * (G + 1) + j;  // the row record
  const ET* lrow = reinterpret_cast<const ET*>(a.logits) + (size_t)rq.trow * (size_t)V;
  const bool draft_pos = j < rq.gamma;
  const bool req_q = rq.q0 >= 0;  // the request carries draft rows
  const bool has_q = req_q && draft_pos;
  const float* qrow = has_q ? a.q + ((size_t)rq.q0 + j) * (size_t)V : nullptr;
  const float T = uni(rq.T);
  const Scale2 c = uni_s2(target_scale(T));
  const DraftW dw = uni_dw(draft_w(T));
  const bool temper = T != 1.f;
  const bool filt = rq.kact || rq.pact;
  const bool cand = rq.kact && rq.k <= kKFast;

  // the draft token's logit and probability, loaded before the stream
  int y = -1;
  float ly = 0.f, qyv = 0.f;
  if (tid == 0 && draft_pos) {
    y = a.ids[(size_t)rq.id0 + j];
    ly = LT::at(lrow, (size_t)y);
    if (req_q) qyv = F32::at(qrow, (size_t)y);
    if (TOK) {
      ly = tok_logit<LT>(tk, y, ly);
      qyv = tok_prob(tk, y, qyv);
    }
  }

  StochState st;
  st.m = cand ? -INFINITY : -FLT_MAX;
  st.z = 0.0;
  st.r = 0.0;
  st.qinv = scale_inv(1);
  st.qbad = 0u;
  st.lbad = 0u;
  st.ps = ChunkState{0, 0u, 0};
  st.qs = ChunkState{0, 0u, 0};
  const int qm = has_q ? (temper ? ((dw.precise && !cand) ? 3 : 2) : 1) : 0;
  if (cand) {
    if (qm == 0) stream_stochastic<LT, VEC, 0, true, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
    else if (qm == 1) stream_stochastic<LT, VEC, 1, true, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
    else stream_stochastic<LT, VEC, 2, true, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
    // each wave cuts its own buffers down to its k-th largest chunk key and
    // copies the tokens at or above that threshold into its segment
    __builtin_amdgcn_s_setprio(2);
    if (st.ps.cnt > rq.k && !st.ps.ovf)
      st.ps = chunk_refresh((LDS_AS ChunkBuf<typename LT::Raw>*)&sh.pb[wave], st.ps, rq.k, 0);
    if (has_q && st.qs.cnt > rq.k && !st.qs.ovf)
      st.qs = chunk_refresh((LDS_AS ChunkBuf<F32::Raw>*)&sh.qb[wave], st.qs, rq.k, 0);
    __builtin_amdgcn_s_setprio(2);
    int n = st.ps.ovf ? kSeg + 1
                      : gather_tokens((const LDS_AS ChunkBuf<typename LT::Raw>*)&sh.pb[wave], st.ps.cnt, st.ps.thr, V,
                                      (LDS_AS uint32_t*)&sh.skey[0][wave * kSeg], (LDS_AS int*)&sh.sid[0][wave * kSeg]);
    if (lane == 0) sh.scnt[0][wave] = n;
    if (has_q) {
      n = st.qs.ovf ? kSeg + 1
                    : gather_tokens((const LDS_AS ChunkBuf<F32::Raw>*)&sh.qb[wave], st.qs.cnt, st.qs.thr, V,
                                    (LDS_AS uint32_t*)&sh.skey[1][wave * kSeg], (LDS_AS int*)&sh.sid[1][wave * kSeg]);
      if (lane == 0) sh.scnt[1][wave] = n;
    }
  } else {
    if (qm == 0) stream_stochastic<LT, VEC, 0, false, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
    else if (qm == 1) stream_stochastic<LT, VEC, 1, false, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
    else if (qm == 2) stream_stochastic<LT, VEC, 2, false, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
    else stream_stochastic<LT, VEC, 3, false, TOK>(lrow, qrow, V, c, dw, rq.k, sh, st, tk);
  }

  // the rest of the row is short serial work that holds this workgroup's
  // slot: issue it ahead of other workgroups' streaming waves
  __builtin_amdgcn_s_setprio(2);
  // ---- block totals: two exchanges, combined in a fixed order ----
  {
    const float mw = wave_max_f32(st.m);
    const uint32_t qbw = has_q ? wave_max_u32(st.qbad) : 0u;
    const uint32_t lbw = cand ? wave_max_u32(st.lbad) : 0u;
    double rt = st.r;
    if (has_q && !cand && temper && rt != 0.0 && scale_e(st.qbad) != scale_e(qbw))
      rt *= scale_step(scale_e(st.qbad), scale_e(qbw), dw.invT);
    const double rw = (has_q && !cand) ? wave_sum_f64(rt) : 0.0;
    if (lane == 0) {
      sh.xm[wave] = mw;
      sh.xqb[wave] = qbw;
      sh.xlb[wave] = lbw;
      sh.xr[wave] = rw;
      sh.ps[wave] = st.ps;
      sh.qs[wave] = st.qs;
    }
  }
  __syncthreads();
  const float m = __builtin_fmaxf(__builtin_fmaxf(sh.xm[0], sh.xm[1]), __builtin_fmaxf(sh.xm[2], sh.xm[3]));
  const uint32_t qb = max(max(sh.xqb[0], sh.xqb[1]), max(sh.xqb[2], sh.xqb[3]));
  // the draft weight scale qs of the row (1 where the weights are q itself)
  const float qinv = (has_q && temper) ? scale_inv(scale_e(qb)) : 1.f;
  double xr[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    xr[w] = sh.xr[w];
    if (has_q && !cand && temper && xr[w] != 0.0 && scale_e(sh.xqb[w]) != scale_e(qb))
      xr[w] *= scale_step(scale_e(sh.xqb[w]), scale_e(qb), dw.invT);
  }
  const double R = (xr[0] + xr[1]) + (xr[2] + xr[3]);
  const uint32_t lb = max(max(sh.xlb[0], sh.xlb[1]), max(sh.xlb[2], sh.xlb[3]));
  if (cand) {
    // a segment that overflowed is gathered again with the largest wave
    // threshold, which keeps far fewer tokens
    const bool p_over = (sh.scnt[0][0] > kSeg) | (sh.scnt[0][1] > kSeg) | (sh.scnt[0][2] > kSeg) | (sh.scnt[0][3] > kSeg);
    const bool q_over = has_q && ((sh.scnt[1][0] > kSeg) | (sh.scnt[1][1] > kSeg) | (sh.scnt[1][2] > kSeg) |
                                  (sh.scnt[1][3] > kSeg));
    if (p_over || q_over) {
      const int np = sh.scnt[0][wave], nq = has_q ? sh.scnt[1][wave] : 0;
      __syncthreads();
      if (np > kSeg) {
        uint32_t L = 0u;
        int ovf = 0;
        for (int w = 0; w < kWaves; ++w) {
          L = max(L, sh.ps[w].thr);
          ovf |= sh.ps[w].ovf;
        }
        const int n = ovf ? kSeg + 1
                          : gather_tokens((const LDS_AS ChunkBuf<typename LT::Raw>*)&sh.pb[wave], st.ps.cnt, L, V,
                                          (LDS_AS uint32_t*)&sh.skey[0][wave * kSeg], (LDS_AS int*)&sh.sid[0][wave * kSeg]);
        if (lane == 0) sh.scnt[0][wave] = n;
      }
      if (nq > kSeg) {
        uint32_t L = 0u;
        int ovf = 0;
        for (int w = 0; w < kWaves; ++w) {
          L = max(L, sh.qs[w].thr);
          ovf |= sh.qs[w].ovf;
        }
        const int n = ovf ? kSeg + 1
                          : gather_tokens((const LDS_AS ChunkBuf<F32::Raw>*)&sh.qb[wave], st.qs.cnt, L, V,
                                          (LDS_AS uint32_t*)&sh.skey[1][wave * kSeg], (LDS_AS int*)&sh.sid[1][wave * kSeg]);
        if (lane == 0) sh.scnt[1][wave] = n;
      }
      __syncthreads();
    }
  }
  // without top-k: Z = sum over the row; with it the kept mass is found below
  double Z = 1.0;
  if (!cand) {
    const double zw = wave_sum_f64(st.z * exp2(((double)st.m - (double)m) * c.d));
    if (lane == 0) sh.xz[wave] = zw;
    __syncthreads();
    Z = (sh.xz[0] + sh.xz[1]) + (sh.xz[2] + sh.xz[3]);
  }
  int fault = 0;
  if (cand ? (lb > 0x7f800000u || !isfinite(m)) : (!(Z > 0.0) || isinf(Z))) fault |= kFaultTargetRow;
  if (has_q && qb >= 0x7f800000u) fault |= kFaultDraftRow;

  float cut_p = -INFINITY, cut_q = -INFINITY;
  double Zk = Z, Rk = R;
  MergeOut mp;  // target top-k set left in LDS by the merge (mp.ok)
  mp.ok = 0;
  if (!fault && filt) {
    bool pdone = false, qdone = !has_q;
    if (cand) {
      // wave 0 merges the target buffers, wave 1 the draft buffers
      if (wave < (has_q ? 2 : 1)) {
        const int d = wave;
        MergeIn in;
        in.L = 0u;
        in.ovf = 0;
        for (int w = 0; w < kWaves; ++w) {
          const ChunkState cs = d == 0 ? sh.ps[w] : sh.qs[w];
          in.L = max(in.L, cs.thr);
          in.ovf |= cs.ovf;
        }
        in.k = rq.k;
        in.top_p = rq.p;
        in.pact = rq.pact;
        in.draft = d;
        in.m = m;
        in.cd = c.d;
        in.T = T;
        in.qinv = qinv;
        MergeOut mo;
        if (d == 0)
          mo = wave_merge<sizeof(ET) == 2>(in, (LDS_AS uint32_t*)sh.skey[0], (LDS_AS int*)sh.sid[0],
                                           (const LDS_AS int*)sh.scnt[0], (LDS_AS double*)sh.pb);
        else
          mo = wave_merge<false>(in, (LDS_AS uint32_t*)sh.skey[1], (LDS_AS int*)sh.sid[1],
                                 (const LDS_AS int*)sh.scnt[1], (LDS_AS double*)sh.qb);
        if (lane == 0) sh.mo[d] = mo;
      }
      __syncthreads();
      mp = sh.mo[0];
      if (mp.ok) {
        pdone = true;
        cut_p = mp.cut;
        Zk = mp.mass;
      }
      if (has_q) {
        const MergeOut mq = sh.mo[1];
        if (mq.ok) {
          qdone = true;
          cut_q = mq.cut;
          Rk = mq.mass;
        }
      }
    }
    if (!pdone) {
      GeneralArgs g;
      g.row = lrow;
      g.V = V;
      g.bf16 = sizeof(ET) == 2;
      g.draft = false;
      g.m = m;
      g.T = T;
      g.qinv = 1.f;
      g.temper = temper;
      g.k = rq.k;
      g.kact = rq.kact;
      g.top_p = rq.p;
      g.pact = rq.pact;
      g.total = Z;
      const Filtered f = general_filter(g, (LDS_AS double*)sh.pb, (LDS_AS double*)sh.sel_d,
                                        (LDS_AS uint32_t*)sh.sel_u, (LDS_AS double*)sh.red_d, tk.ban, TOK ? tk.nban : 0,
                                        tk.pid, tk.pd, TOK == 2 ? tk.npen : 0, tk.theta);
      cut_p = f.cut;
      Zk = f.mass;
    }
    if (!qdone) {
      GeneralArgs g;
      g.row = qrow;
      g.V = V;
      g.bf16 = false;
      g.draft = true;
      g.m = m;
      g.T = T;
      g.qinv = qinv;
      g.temper = temper;
      g.k = rq.k;
      g.kact = rq.kact;
      g.top_p = rq.p;
      g.pact = rq.pact;
      g.total = R;
      // (histogram in the draft buffers: the target weights stay for the draw)
      const Filtered f = general_filter(g, (LDS_AS double*)sh.qb, (LDS_AS double*)sh.sel_d,
                                        (LDS_AS uint32_t*)sh.sel_u, (LDS_AS double*)sh.red_d, tk.ban, TOK ? tk.nban : 0,
                                        tk.pid, tk.pd, TOK == 2 ? tk.npen : 0, tk.theta);
      cut_q = f.cut;
      Rk = f.mass;
    }
  }
  if (!fault && has_q && !(Rk > 0.0)) fault |= kFaultDraftMass;

  if (wave == 0) {
    // accept flag (thread 0 holds the draft token's values), then, if this row
    // can be the one the request draws from (the bonus row, or a rejected
    // draft row), the draw itself from the kept list still in LDS
    RowStats s;
    s.m = m;
    s.cut_p = cut_p;
    s.cut_q = cut_q;
    s.qinv = qinv;
    s.z = Zk;
    s.r = Rk;
    s.p_y = NAN;
    s.q_y = NAN;
    int acc = 0;
    if (lane == 0 && draft_pos && !fault) {
      const double e = (ly >= cut_p) ? mass_p(ly, m, c) : 0.0;
      const double py = e / Zk;
      double qy = 1.0;
      if (req_q) qy = (qyv >= cut_q) ? temper_q(qyv, T, qinv) / Rk : 0.0;
      const double u = (double)a.u_accept[(size_t)rq.id0 + j];
      acc = (!a.synthetic && u * qy < py) ? 1 : 0;  // synthetic mode: the listed draft row is A
      s.p_y = py;
      s.q_y = qy;
    }
    acc = __builtin_amdgcn_readlane(acc, 0);
    DrawOut d;
    d.z = -1;
    d.s = NAN;
    if (!fault && mp.ok && !(draft_pos && acc)) {
      DrawIn din;
      din.nk = mp.nk;
      din.cutkey = mp.cutkey;
      din.zk = Zk;
      din.mode = draft_pos ? (has_q ? 1 : 2) : 0;
      din.qrow = qrow;
      din.cut_q = cut_q;
      din.T = T;
      din.qinv = qinv;
      din.rk = Rk;
      din.y = __builtin_amdgcn_readlane(y, 0);
      din.us = a.u_sample[i];
      d = wave_draw(din, (const LDS_AS uint32_t*)sh.skey[0], (const LDS_AS int*)sh.sid[0],
                    (const LDS_AS double*)sh.pb, (LDS_AS double*)sh.qb, tk.ban, TOK ? tk.nban : 0, tk.pid,
                    tk.pd, TOK == 2 ? tk.npen : 0);
    }
    if (lane == 0) {
      s.s = d.s;
      s.flags = acc | (fault << 8);
      s.draw = d.z;
      publish(a.stats + row, s);
      note_row(a, i, j, acc, fault, d.z < 0);
    }
  }
}

// ------------------------------------------------------------------------------------------
// kernels
// ------------------------------------------------------------------------------------------

// One workgroup: writes each request's record (gamma_i, where its rows and
// drafts sit in the inputs, cleared outcome bits) and lists the draft rows
// (request i, position j < gamma_i) request-major, so that the row pass
// launches no workgroup for a padding position.  Padded layout: gamma_i is
// the index of the first negative draft id.  Flattened layout: gamma_i =
// cu[i] - cu[i-1]; a count outside [0, G] (or past T) faults the request,
// which then lists no draft rows; the draft-probability rows of the requests
// that carry them are consecutive, so request i's first one is the sum of
// gamma_r over the earlier such requests (a second prefix sum).
__global__ __launch_bounds__(kBlock) void plan_kernel(Args a) {
  __shared__ int s_scan[2][kWaves];
  __shared__ int s_base[2];
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int kPer = 4;  // requests per thread and round
  if (tid < 2) s_base[tid] = 0;
  if (tid == 0) *a.nfault = 0u;  // the draw pass counts this call's faulted requests
  __syncthreads();
  for (int r0 = 0; r0 < a.N; r0 += kBlock * kPer) {
    int gam[kPer], nl[kPer], gq[kPer], id0[kPer];
    unsigned int lf[kPer];
    bool hq[kPer];
    int cnt = 0, qcnt = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = r0 + tid * kPer + u;
      gam[u] = nl[u] = gq[u] = id0[u] = 0;
      lf[u] = 0u;
      hq[u] = false;
      if (i < a.N) {
        if (a.cu) {
          const int prev = i ? a.cu[i - 1] : 0, cur = a.cu[i];
          const long long g = (long long)cur - prev;
          id0[u] = prev;
          hq[u] = a.q && (!a.has_q || a.has_q[i]);
          if (prev < 0 || g < 0 || g > a.G || cur > a.T) lf[u] = kFaultDraftCount;
          else gam[u] = (int)g;
          // later requests' draft-probability rows sit after this one's, whatever its count
          gq[u] = (hq[u] && g > 0) ? (int)min(g, (long long)a.T) : 0;
        } else {
          int g = a.G;
          for (int jj = a.G - 1; jj >= 0; --jj)
            if (a.ids[(size_t)i * a.G + jj] < 0) g = jj;
          gam[u] = g;
          id0[u] = i * a.G;
          hq[u] = a.q != nullptr;
        }
        // rows listed: the draft rows; in the synthetic mode only row A (the bonus
        // rows of the standard mode are launched after the listed ones)
        nl[u] = a.synthetic ? 1 : gam[u];
      }
      cnt += nl[u];
      qcnt += gq[u];
    }
    // exclusive offsets: wave scans, then the four wave totals
    const int incl = wave_incl_scan_i32(cnt);
    const int qincl = wave_incl_scan_i32(qcnt);
    if (lane_id() == 63) {
      s_scan[0][wave] = incl;
      s_scan[1][wave] = qincl;
    }
    __syncthreads();
    int off = s_base[0] + incl - cnt, qoff = s_base[1] + qincl - qcnt;
    for (int w = 0; w < wave; ++w) {
      off += s_scan[0][w];
      qoff += s_scan[1][w];
    }
    const int round_total = s_scan[0][0] + s_scan[0][1] + s_scan[0][2] + s_scan[0][3];
    const int qround_total = s_scan[1][0] + s_scan[1][1] + s_scan[1][2] + s_scan[1][3];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = r0 + tid * kPer + u;
      if (i < a.N) {
        // synthetic mode: draft j is accepted iff u_j < rate_j, so the first
        // rejection A is known before any row is read
        int As = gam[u];
        if (a.synthetic)
          for (int jj = 0; jj < gam[u]; ++jj)
            if (!(a.u_accept[(size_t)id0[u] + jj] < a.srates[jj])) {
              As = jj;
              break;
            }
        ReqRec r;
        r.acc = !a.synthetic ? 0ull : (As >= 64 ? ~0ull : ((1ull << As) - 1ull));
        r.nodraw = 0ull;
        r.nodraw64 = 0u;
        r.fault = 0u;
        r.gamma = gam[u];
        r.tgt0 = a.cu ? id0[u] + i : i * (a.G + 1);
        r.id0 = id0[u];
        r.q0 = !hq[u] ? -1 : (a.cu ? qoff : i * a.G);
        r.lfault = lf[u];
        r.pad = 0;
        a.rec[i] = r;
        if (a.synthetic) a.plan[1 + off] = i * 128 + As;
        else
          for (int jj = 0; jj < gam[u]; ++jj) a.plan[1 + off + jj] = i * 128 + jj;
      }
      off += nl[u];
      qoff += gq[u];
    }
    __syncthreads();
    if (tid == 0) {
      s_base[0] += round_total;
      s_base[1] += qround_total;
    }
    __syncthreads();
  }
  if (tid == 0) a.plan[0] = s_base[0];
}

// presence / frequency part of a listed token's delta (count > 0), each
// operation rounded to float32
__device__ inline float pen_delta(float freq, int cnt, float pres) {
#pragma clang fp contract(off)
  const float f = freq * (float)cnt;
  return f + pres;
}

// Position j of request i: its penalty list into LDS (ids, deltas), the
// request's repetition penalty, and every staging slot set to NaN.  With `check` (the row pass) the
// list and the penalties are validated: at most kPenMax ids, strictly
// ascending, in [0, V), counts >= 0; a positive finite repetition penalty,
// finite presence and frequency penalties, and a repetition penalty of 1 on a
// request that carries draft rows and samples (its draft probabilities fix
// the draft's logits only up to a constant).  Returns the list length, or -1
// when a check fails.  Every thread of the workgroup calls it.
__device__ inline int load_penalties(const Args& a, const Req& rq, int i, int j, LDS_AS int* pid, LDS_AS float* pd,
                                     LDS_AS float* stage, float& theta, bool check) {
  const int pos = rq.id0 + i + j;  // the position's index in the flattened layout
  const int p0 = a.pen_off[pos], n = a.pen_off[pos + 1] - p0;
  theta = a.pen_rep ? a.pen_rep[i] : 1.f;
  const float pres = a.pen_pres ? a.pen_pres[i] : 0.f, freq = a.pen_freq ? a.pen_freq[i] : 0.f;
  int bad = 0;
  if (check)
    bad = (n < 0 || n > kPenMax || (n > 0 && (!a.pen_ids || !a.pen_cnt)) || !(theta > 0.f) || isinf(theta) ||
           !isfinite(pres) || !isfinite(freq) || (theta != 1.f && rq.q0 >= 0 && !rq.greedy))
              ? 1
              : 0;
  if (!bad)
    for (int t = threadIdx.x; t < n; t += kBlock) {
      const int id = a.pen_ids[(size_t)p0 + t], cnt = a.pen_cnt[(size_t)p0 + t];
      const float d = cnt > 0 ? pen_delta(freq, cnt, pres) : 0.f;
      pid[t] = id;
      pd[t] = d;
      if (check) bad |= (id < 0 || id >= a.V || cnt < 0 || (t > 0 && a.pen_ids[(size_t)p0 + t - 1] >= id)) ? 1 : 0;
    }
  for (int t = threadIdx.x; t < kWaves * 512; t += kBlock) stage[t] = __uint_as_float(0x7fffffffu);
  bad = __syncthreads_or(bad);
  return bad ? -1 : n;
}

template <class LT, bool VEC, int TOK>
__global__ __launch_bounds__(kBlock, TOK == 2 ? 2 : (sizeof(typename LT::T) == 2 ? 3 : 2)) void row_kernel(Args a) {
  __shared__ RowShared<LT> sh;
  __shared__ int s_ban[TOK ? kBanMax : 1];
  __shared__ int s_pid[TOK == 2 ? kPenMax : 1];
  __shared__ float s_pd[TOK == 2 ? kPenMax : 1];
  __shared__ float s_stage[TOK == 2 ? kWaves * 512 : 1];
  // The draft rows first (the larger rows), request-major (consecutive
  // blocks, which dispatch round-robin over the 8 XCDs, read neighbouring
  // rows, in memory order), then one bonus row per request.  Plan mode: the
  // plan lists the draft rows and the launch's blocks past the real rows exit
  // at once.  Direct mode: request i owns `dslots` consecutive blocks, slot
  // j < gmax being position j (a padding position exits at once).  With
  // gmax a multiple of 8 there is one more slot, which exits without a load:
  // otherwise block i * gmax + j would sit on XCD j for every request, and a
  // ragged batch's mostly-padding high positions would leave XCDs idle.
  const int bx = (int)blockIdx.x;
  int i, j;
  Req rq;
  if (a.direct) {
    if (bx == 0 && threadIdx.x == 0) *a.nfault = 0u;  // the find kernel counts this call's faulted requests
    const int ns = a.dslots;
    const int nd = a.N * ns;
    const bool bonus = bx >= nd;
    i = bonus ? bx - nd : bx / ns;
    const int slot = bonus ? 0 : bx - i * ns;
    if (!bonus && slot >= a.G) return;
    rq = load_req(a, i);
    j = bonus ? rq.gamma : slot;
    if (!bonus && j >= rq.gamma) return;
  } else {
    const int nd = a.plan[0];
    if (bx >= nd + (a.synthetic ? 0 : a.N)) return;
    const bool bonus = bx >= nd;
    const int m = bonus ? 0 : a.plan[1 + bx];
    i = bonus ? bx - nd : (m >> 7);
    rq = load_req(a, i);
    j = bonus ? rq.gamma : (m & 127);
  }
  // the row's place in target_logits: request order, or the caller's indices
  rq.trow = (long long)rq.tgt0 + j;
  if (a.bidx && !rq.fault) {
    const int r = j < rq.gamma ? a.tidx[(size_t)rq.id0 + j] : a.bidx[i];
    if (r < 0 || r >= a.R) rq.fault |= kFaultRowIndex;
    rq.trow = r;
  }
  int nban = 0;
  if (TOK && a.ban_off) {
    // the request's banned tokens into LDS: at most kBanMax, strictly
    // ascending, each in [0, V); otherwise the request faults
    const int b0 = a.ban_off[i], n = a.ban_off[i + 1] - b0;
    int bad = (n < 0 || n > kBanMax || (n > 0 && !a.ban_ids)) ? 1 : 0;
    if (!bad)
      for (int t = threadIdx.x; t < n; t += kBlock) {
        const int id = a.ban_ids[(size_t)b0 + t];
        s_ban[t] = id;
        bad |= (id < 0 || id >= a.V || (t > 0 && a.ban_ids[(size_t)b0 + t - 1] >= id)) ? 1 : 0;
      }
    bad = __syncthreads_or(bad);
    if (bad) rq.fault |= kFaultBanList;
    else nban = n;
  }
  int npen = 0;
  float theta = 1.f;
  // (a request whose draft count is out of range has no valid positions)
  if (TOK == 2 && !(rq.fault & kFaultDraftCount)) {
    npen = load_penalties(a, rq, i, j, (LDS_AS int*)s_pid, (LDS_AS float*)s_pd, (LDS_AS float*)s_stage, theta, true);
    if (npen < 0) rq.fault |= kFaultPenalty;
  }
  if (rq.fault) {
    if (threadIdx.x == 0) {
      if (a.direct) {
        RowStats s;
        s.m = NAN;
        s.cut_p = -INFINITY;
        s.cut_q = -INFINITY;
        s.argmax = -1;
        s.z = s.r = s.p_y = s.q_y = s.s = NAN;
        s.flags = rq.fault << 8;
        s.draw = -1;
        publish(a.stats + (size_t)i * (a.G + 1) + j, s);
      }
      note_row(a, i, j, 0, rq.fault, false);
    }
    return;
  }
  const Toks tk = toks((const LDS_AS int*)s_ban, nban, (const LDS_AS int*)s_pid, (const LDS_AS float*)s_pd,
                       (LDS_AS float*)s_stage + (threadIdx.x >> 6) * 512, npen, theta);
  if (rq.greedy) greedy_row<LT, VEC, TOK>(a, rq, i, j, sh, tk);
  else stochastic_row<LT, VEC, TOK>(a, rq, i, j, sh, tk);
}

// ------------------------------------------------------------------------------------------
// draw pass: requests whose draw row had no kept list in LDS
// ------------------------------------------------------------------------------------------

// Inclusive prefix sum of doubles over a full wave.
__device__ inline double wave_incl_scan_f64(double v) {
  v += dpp_add_src<0x111, 0xF>(v);  // row_shr:1
  v += dpp_add_src<0x112, 0xF>(v);  // row_shr:2
  v += dpp_add_src<0x114, 0xF>(v);  // row_shr:4
  v += dpp_add_src<0x118, 0xF>(v);  // row_shr:8
  v += dpp_add_src<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_add_src<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

// What the draw pass needs to weigh row A's tokens.
struct DrawW {
  float m;          // max logit of the row
  float cut_p;      // target token kept iff logit >= cut_p
  float cut_q;      // draft token kept iff q >= cut_q
  float qinv;       // 1 / qs of the tempered draft weights
  float invZf;      // 1 / kept target mass, fp32
  float invRf;      // 1 / kept draft mass, fp32
  Scale2 c;         // log2(e) / T
  DraftW dw;        // tempered draft weights
  double invZ;      // 1 / kept target mass, fp64 (weights formed in fp64)
  double invR;      // 1 / kept draft mass, fp64
  bool temper;      // T != 1
  int mode;         // 0: p'; 1: max(0, p' - q'); 2: p' with the draft token removed
  int yA;           // mode 2: the draft token
};

// wave-uniform copies (scalar registers) of the draw parameters
__device__ inline DrawW uni_draw(DrawW d) {
  d.m = uni(d.m);
  d.cut_p = uni(d.cut_p);
  d.cut_q = uni(d.cut_q);
  d.qinv = uni(d.qinv);
  d.invZf = uni(d.invZf);
  d.invRf = uni(d.invRf);
  d.c = uni_s2(d.c);
  d.dw = uni_dw(d.dw);
  d.invZ = uni(d.invZ);
  d.invR = uni(d.invR);
  d.temper = uni((int)d.temper);
  d.mode = uni(d.mode);
  d.yA = uni(d.yA);
  return d;
}

// Draw weight of token x (lv its logit, qv its draft probability) under draw
// mode MODE (0: p'; 1: max(0, p' - q'); 2: p' with the draft token's cell
// removed); tokens past the row end read as -inf logits and zero
// probabilities, so their weight is zero.  The exponents are formed as in the
// row pass's sums, so that each p' is its weight over the very sum that
// weight entered; p' - q' is one fused multiply-add.  TEMPER: T != 1.  FILT:
// the row kept a top-k / top-p set (cuts above -inf); without one every
// token is kept, the row pass having faulted any NaN or negative value.
// PRECISE (a tempered residual at 1/T above kPreciseInvT): the draft weights
// that carry mass are formed in fp64 as in the row pass, then normalised and
// subtracted in fp64.  Contraction is off, so every caller forms the same
// weight.
template <int MODE, bool TEMPER, bool FILT, bool PRECISE>
__device__ inline float draw_w(float lv, float qv, int x, const DrawW& d) {
#pragma clang fp contract(off)
  float e = mass_p32(lv, d.m, d.c);
  if (FILT && !(lv >= d.cut_p)) e = 0.f;
  if (MODE == 1) {
    float r = qv;
    if (TEMPER) {
      const float rr = qv * d.qinv;
      const float xq = smul(fast_log2(rr), d.dw.invT);
      if (PRECISE && xq > d.dw.thr && (!FILT || qv >= d.cut_q)) {
        const double w = (double)e * d.invZ - precise_weight_call(rr, d.dw.invT.d) * d.invR;
        return w > 0.0 ? (float)w : 0.f;
      }
      r = fast_exp2(xq);
    }
    float q = r * d.invRf;
    if (FILT && !(qv >= d.cut_q)) q = 0.f;
    return __builtin_fmaxf(__builtin_fmaf(e, d.invZf, -q), 0.f);
  }
  const float p = e * d.invZf;
  if (MODE == 2) return x == d.yA ? 0.f : p;
  return p;
}

// The same weight with the mode chosen at run time (the find kernel, one
// block per request); FILT = true equals FILT = false on rows without a cut.
template <bool PRECISE>
__device__ inline float draw_weight(float lv, float qv, int x, const DrawW& d) {
  if (d.mode == 1)
    return d.temper ? draw_w<1, true, true, PRECISE>(lv, qv, x, d) : draw_w<1, false, true, false>(lv, qv, x, d);
  if (d.mode == 2) return draw_w<2, false, true, false>(lv, qv, x, d);
  return draw_w<0, false, true, false>(lv, qv, x, d);
}

// A lane's 8 weights summed pairwise in fp32 (the row pass sums its exponent
// terms the same way), widened to fp64 for the block and row sums; the fp64
// weights of the precise form are summed in fp64, in token order.
__device__ inline double lane_sum8(const float w[8]) {
  return (double)(((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7])));
}
__device__ inline double lane_sum8_seq(const float w[8]) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += (double)w[e];
  return s;
}

// Request i's outputs from its record: the accepted drafts before the first
// rejection A, the token at A (drawn in the row pass, or a greedy row's
// argmax; left to the draw below when `defer`), -1 after it, and the
// diagnostics.  Run by one workgroup per request.
// In direct mode (`lanes`) lane t of each wave already holds draft id t
// (lid) and row t's draw (ldr; row 64's in dr64) from rebuilding the record,
// so the outputs need no loads of their own.
__device__ inline void request_outputs(const Args& a, int i, const ReqRec& rr, int A, bool defer, bool lanes,
                                       int lid, int ldr, int dr64) {
  const int G = a.G, tid = threadIdx.x;
  int32_t* out = a.out_tokens + (size_t)i * (G + 1);
  const RowStats* st = a.stats + (size_t)i * (G + 1);
  const unsigned int fault = rr.fault | rr.lfault;
  if (fault) {
    for (int t = tid; t <= G; t += kBlock) out[t] = -1;
    if (tid == 0) {
      __hip_atomic_fetch_add(a.nfault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.out_num[i] = -1;
      if (a.d_fault) a.d_fault[i] = (int)fault;
      if (a.d_resid) a.d_resid[i] = NAN;
    }
    if (a.d_py)
      for (int t = tid; t < G; t += kBlock) a.d_py[(size_t)i * G + t] = NAN;
    if (a.d_qy)
      for (int t = tid; t < G; t += kBlock) a.d_qy[(size_t)i * G + t] = NAN;
    return;
  }
  int z = -1;
  double S = NAN;
  if (!defer) {
    z = lanes ? (A < 64 ? __builtin_amdgcn_readlane(ldr, A) : dr64) : st[A].draw;
    if (a.d_resid) S = st[A].s;
  }
  for (int t = tid; t <= G; t += kBlock) {
    if (defer && t == A) continue;
    // (t < 64: this thread is lane t of wave 0)
    out[t] = t < A ? ((lanes && t < 64) ? lid : a.ids[(size_t)rr.id0 + t]) : (t == A ? z : -1);
  }
  if (tid == 0) {
    a.out_num[i] = A;
    if (a.d_fault) a.d_fault[i] = 0;
    if (a.d_resid && !defer) a.d_resid[i] = S;
  }
  if (a.d_py || a.d_qy) {
    for (int t = tid; t < G; t += kBlock) {
      const bool real = t < rr.gamma && !a.synthetic;
      if (a.d_py) a.d_py[(size_t)i * G + t] = real ? st[t].p_y : NAN;
      if (a.d_qy) a.d_qy[(size_t)i * G + t] = real ? st[t].q_y : NAN;
    }
  }
}

// Where request i's draw happens: its record, the first rejection A, whether
// row A left the draw to this pass, and where row A sits.  The record and the
// request's temperature are loaded together.
template <class LT>
struct DrawCtx {
  ReqRec rr;
  int A, mode, nsteps;
  bool defer;
  float T;
  const typename LT::T* lrow;
  const float* qrow;
  DrawSum* ds;  // [nsteps * kWaves] block sums of row A
  bool lanes;   // direct mode: lane t holds draft id t and row t's draw
  int lid, ldr, ldr64;
};

// Direct mode: request i's record rebuilt from its draft ids (gamma_i: the
// first negative one) and its rows' records (accept flag, fault bits, whether
// the row drew), one load of each per lane; row 64 (gmax = 64) separately.
__device__ inline ReqRec direct_rec(const Args& a, int i, int& lid, int& ldr, int& ldr64) {
  const int lane = lane_id(), G = a.G;
  const RowStats* st = a.stats + (size_t)i * (G + 1);
  const int id = lane < G ? a.ids[(size_t)i * G + lane] : 0;
  const int fl = lane <= G ? st[lane].flags : 0;
  const int dr = lane <= G ? st[lane].draw : 0;
  const int fl64 = G == 64 ? st[64].flags : 0;
  const int dr64 = G == 64 ? st[64].draw : 0;
  const uint64_t neg = __ballot(lane < G && id < 0);
  ReqRec r;
  r.gamma = neg ? __ffsll((unsigned long long)neg) - 1 : G;
  const int gamma = r.gamma;
  r.acc = __ballot(lane < gamma && (fl & 1));
  r.nodraw = __ballot(lane <= gamma && dr < 0);
  r.nodraw64 = (gamma == 64 && dr64 < 0) ? 1u : 0u;
  int f = lane <= gamma ? (fl >> 8) : 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) f |= __shfl_xor(f, o);
  r.fault = (unsigned int)(__builtin_amdgcn_readfirstlane(f) | (gamma == 64 ? (fl64 >> 8) : 0));
  r.tgt0 = i * (G + 1);
  r.id0 = i * G;
  r.q0 = a.q ? i * G : -1;
  r.lfault = 0u;
  r.pad = 0;
  lid = id;
  ldr = dr;
  ldr64 = dr64;
  return r;
}

template <class LT>
__device__ inline DrawCtx<LT> draw_ctx(const Args& a, int i) {
  typedef typename LT::T ET;
  DrawCtx<LT> x;
  x.lanes = a.direct != 0;
  x.lid = x.ldr = x.ldr64 = 0;
  if (a.direct) x.rr = direct_rec(a, i, x.lid, x.ldr, x.ldr64);
  else x.rr = a.rec[i];
  x.T = a.temperature ? a.temperature[i] : 1.f;
  const ReqRec& rr = x.rr;
  const int gamma = rr.gamma;
  const uint64_t within = gamma >= 64 ? ~0ull : ((1ull << gamma) - 1ull);
  const uint64_t rej = ~rr.acc & within;
  x.A = rej ? (__ffsll((unsigned long long)rej) - 1) : gamma;
  const int A = x.A;
  x.defer = !(rr.fault | rr.lfault) && (A >= 64 ? rr.nodraw64 != 0u : ((rr.nodraw >> A) & 1ull) != 0ull);
  x.mode = A < gamma ? (rr.q0 >= 0 ? 1 : 2) : 0;
  x.nsteps = (a.V + kStep - 1) / kStep;
  x.ds = a.dsum + (size_t)i * x.nsteps * kWaves;
  x.lrow = nullptr;
  x.qrow = nullptr;
  if (!x.defer) return x;
  // (row A's index was checked by the row pass: a bad one faults the request)
  const size_t trow = !a.bidx ? (size_t)rr.tgt0 + A : (size_t)(A < gamma ? a.tidx[(size_t)rr.id0 + A] : a.bidx[i]);
  x.lrow = reinterpret_cast<const ET*>(a.logits) + trow * (size_t)a.V;
  x.qrow = (x.mode == 1) ? a.q + ((size_t)rr.q0 + A) * (size_t)a.V : nullptr;
  return x;
}

// How row A's tokens are weighed: from row A's statistics (wave-uniform).
template <class LT>
__device__ inline DrawW draw_weights(const Args& a, int i, const DrawCtx<LT>& x, const RowStats& sa) {
  const int A = x.A, mode = x.mode;
  DrawW dwt;
  dwt.m = sa.m;
  dwt.cut_p = sa.cut_p;
  dwt.cut_q = sa.cut_q;
  dwt.temper = x.T != 1.f;
  dwt.qinv = (mode == 1 && dwt.temper) ? sa.qinv : 1.f;
  dwt.c = target_scale(x.T);
  dwt.dw = draft_w(x.T);
  dwt.invZ = 1.0 / sa.z;
  dwt.invR = (mode == 1) ? 1.0 / sa.r : 0.0;
  dwt.invZf = (float)dwt.invZ;
  dwt.invRf = (float)dwt.invR;
  dwt.mode = mode;
  dwt.yA = mode == 2 ? a.ids[(size_t)x.rr.id0 + A] : -1;
  return uni_draw(dwt);
}

// Draw pass, part 1 (grid: dparts workgroups per request, kDrawSpan steps of
// row A each).  Each reads the request's record, finds the first rejection A
// and, if row A made no draw of its own (no kept list in LDS), stores the sum
// of the draw weights of each 512-token block (one wave's tokens of one step)
// of its steps.  Row A's loads start as soon as the record is in: kDrawWin
// steps stay in flight, the first window while row A's statistics and lists
// are read.  The next launch reads the sums: the kernel boundary orders the
// stores before the reads, with no hand-off between workgroups of one launch.
template <class LT, bool VEC, int TOK>
__global__ __launch_bounds__(kBlock, (TOK || !VEC || sizeof(typename LT::T) == 4) ? 4 : 6) void draw_kernel(Args a) {
  typedef typename LT::Raw LR;
  constexpr int kWin = sizeof(typename LT::T) == 2 ? kDrawWin : kDrawWin / 2;  // the same bytes in flight
  __shared__ double s_blk[kDrawSpan * kWaves];
  __shared__ int s_ban[TOK ? kBanMax : 1];
  __shared__ int s_pid[TOK == 2 ? kPenMax : 1];
  __shared__ float s_pd[TOK == 2 ? kPenMax : 1];
  __shared__ float s_stage[TOK == 2 ? kWaves * 512 : 1];
  const int i = blockIdx.x / a.dparts, part = blockIdx.x - i * a.dparts;
  const DrawCtx<LT> cx = draw_ctx<LT>(a, i);
  if (!cx.defer) return;
  const int V = a.V, A = cx.A, mode = cx.mode, nsteps = cx.nsteps;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const ReqRec& rr = cx.rr;
  const typename LT::T* lrow = cx.lrow;
  const float* qrow = cx.qrow;
  DrawSum* ds = cx.ds;
  const int s0 = part * kDrawSpan, cnt = min(kDrawSpan, nsteps - s0);
  // a tempered residual at large 1/T: fp64 draft weights, one step at a time
  const bool precise = mode == 1 && cx.T != 1.f && draft_w(cx.T).precise;
  // Steps that lie wholly inside the row are loaded with unconditional
  // 16-byte loads, so all of a window's loads are in flight together (a load
  // that may fall back to element loads for the row's tail puts a wait for
  // every outstanding load at each of its branches).  The row's partial last
  // step, rows without 16-byte alignment and the precise form go one step at
  // a time through the element-wise path.
  const bool unit = !VEC || precise || (s0 + cnt) * kStep > V;
  typedef std::integral_constant<int, 0> M0;
  typedef std::integral_constant<int, 1> M1;
  typedef std::integral_constant<int, 2> M2;
  typedef std::true_type Y;
  typedef std::false_type N;
  // everything from the first loads on, with the draw mode fixed at compile time
  auto run = [&](auto md) {
    constexpr int M = decltype(md)::value;
    LR lr[kWin];
    F32::Raw qr[kWin];
    if constexpr (VEC) {
      if (!unit) {
        // the first window (past this workgroup's last step: that step again, whose weights are not used)
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
          const int base = (s0 + min(u, cnt - 1)) * kStep + tid * kCh;
          lr[u] = LT::load(lrow + base);
          if (M == 1) qr[u] = F32::load(qrow + base);
        }
      }
    }
    const DrawW dwt = draw_weights<LT>(a, i, cx, a.stats[(size_t)i * (a.G + 1) + A]);
    // the request's banned tokens (checked by the row pass, which faults the
    // request on a bad list)
    int nban = 0;
    if (TOK && a.ban_off) {
      const int b0 = a.ban_off[i];
      nban = a.ban_off[i + 1] - b0;
      for (int t = tid; t < nban; t += kBlock) s_ban[t] = a.ban_ids[(size_t)b0 + t];
      __syncthreads();
    }
    // row A's penalty list (checked by the row pass likewise)
    int npen = 0;
    float theta = 1.f;
    if (TOK == 2) {
      Req rq;
      rq.id0 = rr.id0;
      npen = load_penalties(a, rq, i, A, (LDS_AS int*)s_pid, (LDS_AS float*)s_pd, (LDS_AS float*)s_stage, theta,
                            false);
    }
    const Toks tk = toks((const LDS_AS int*)s_ban, nban, (const LDS_AS int*)s_pid, (const LDS_AS float*)s_pd,
                         (LDS_AS float*)s_stage + (threadIdx.x >> 6) * 512, npen, theta);
    // Sum of one lane's 8 draw weights (raw values l, q of step u) under the
    // compile-time draw form (M, TEMPER, FILT, PRECISE); the lists walk
    // ascending 512-token wave ranges, so steps come in order.
    auto lane_sum = [&](LR& l, F32::Raw& q, int u, BanWalk& bw, PenWalk& pw, auto tp, auto ft, auto pr) {
      const int base = (s0 + u) * kStep + tid * kCh;
      if (TOK == 2) pen_walk(pw, tk, (s0 + u) * kStep + wave * 512, l, q, M == 1);
      if (TOK) {
        const uint32_t m = ban_mask(bw, tk.ban, (s0 + u) * kStep + wave * 512);
        if (m) {
          ban_logits(l, m);
          if (M == 1) ban_apply(q, m, 0u);
        }
      }
      float lv[8], qv[8], w[8];
      LT::unpack(l, lv);
      if (M == 1) F32::unpack(q, qv);
      if constexpr (decltype(pr)::value) {
        // fp64 weights: summed as they come (eight interleaved would not fit the registers)
        double sw = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sw += (double)draw_w<1, true, decltype(ft)::value, true>(lv[e], qv[e], base + e, dwt);
        return sw;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          w[e] = draw_w<M, decltype(tp)::value, decltype(ft)::value, false>(lv[e], M == 1 ? qv[e] : 0.f, base + e,
                                                                            dwt);
        return lane_sum8(w);
      }
    };
    BanWalk bw;
    PenWalk pw;
    if (TOK) bw = ban_start(tk.ban, tk.nban);
    if (TOK == 2) pw = pen_start(tk.npen);
    const bool filt = dwt.cut_p > -INFINITY || dwt.cut_q > -INFINITY;
    // one step at a time, element loads at the row's tail
    auto per_step = [&](auto tp, auto ft, auto pr) {
      for (int u = 0; u < cnt; ++u) {
        const int base = (s0 + u) * kStep + tid * kCh;
        LR l = load_logits<LT, VEC>(lrow, base, V);
        F32::Raw q = M == 1 ? load_probs<VEC>(qrow, base, V) : F32::Raw{};
        const double sw = wave_sum_f64(lane_sum(l, q, u, bw, pw, tp, ft, pr));
        if (lane == 0) s_blk[u * kWaves + wave] = sw;
      }
    };
    // step u is reduced while steps u + 1 .. u + kWin are in flight (block
    // sums go to LDS: a global store here would count against the counter the
    // loads wait on)
    auto stream = [&](auto tp, auto ft) {
#pragma unroll
      for (int u = 0; u < kDrawSpan; ++u) {
        if (u >= cnt) break;
        LR l = lr[u % kWin];
        F32::Raw q = qr[u % kWin];
        if (u + kWin < kDrawSpan) {
          const int base = (s0 + min(u + kWin, cnt - 1)) * kStep + tid * kCh;
          lr[u % kWin] = LT::load(lrow + base);
          if (M == 1) qr[u % kWin] = F32::load(qrow + base);
        }
        const double sw = wave_sum_f64(lane_sum(l, q, u, bw, pw, tp, ft, N{}));
        if (lane == 0) s_blk[u * kWaves + wave] = sw;
      }
    };
    auto forms = [&](auto body) {  // the (TEMPER, FILT) forms of mode M
      if (M == 1 && dwt.temper) {
        if (filt) body(Y{}, Y{});
        else body(Y{}, N{});
      } else {
        if (filt) body(N{}, Y{});
        else body(N{}, N{});
      }
    };
    if constexpr (M == 1) {
      if (precise) {
        if (filt) per_step(Y{}, Y{}, Y{});
        else per_step(Y{}, N{}, Y{});
        return;
      }
    }
    if (unit) {
      forms([&](auto tp, auto ft) { per_step(tp, ft, N{}); });
    } else {
      if constexpr (VEC) forms([&](auto tp, auto ft) { stream(tp, ft); });
    }
  };
  if (mode == 1) run(M1{});
  else if (mode == 2) run(M2{});
  else run(M0{});
  __syncthreads();
  if (tid < cnt * kWaves) {
    DrawSum d;
    d.sw = s_blk[tid];
    ds[(size_t)s0 * kWaves + tid] = d;
  }
}

// Draw pass, part 2 (grid: one workgroup per request): the outputs, and the
// draw left to this pass.  Wave 0 loads every block sum of row A (kFindPer
// consecutive blocks per lane, all in flight), forms S = their sum in token
// order (lane sums, then a wave scan), finds the lane, then the block, where
// the running sum first exceeds u * S, re-reads that block and finds the
// token (inverse CDF over ascending id).  Where rounding leaves no crossing:
// the last block, then the last token, of positive weight.  If the weights
// sum to zero, the same over p', whose block sums the workgroup forms itself.
template <class LT, bool VEC, int TOK>
__global__ __launch_bounds__(kBlock) void find_kernel(Args a) {
  typedef typename LT::Raw LR;
  __shared__ int s_ban[TOK ? kBanMax : 1];
  __shared__ int s_pid[TOK == 2 ? kPenMax : 1];
  __shared__ float s_pd[TOK == 2 ? kPenMax : 1];
  __shared__ float s_stage[TOK == 2 ? kWaves * 512 : 1];
  __shared__ double s_tw;
  const int i = blockIdx.x;
  const DrawCtx<LT> cx = draw_ctx<LT>(a, i);
  const float us = a.u_sample[i];
  request_outputs(a, i, cx.rr, cx.A, cx.defer, cx.lanes, cx.lid, cx.ldr, cx.ldr64);
  if (!cx.defer) return;
  const int G = a.G, V = a.V, A = cx.A, mode = cx.mode, nsteps = cx.nsteps;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const ReqRec& rr = cx.rr;
  const typename LT::T* lrow = cx.lrow;
  const float* qrow = cx.qrow;
  DrawSum* ds = cx.ds;
  const int nb = nsteps * kWaves;
  constexpr int kChunk = 64 * kFindPer;
  // one chunk of block sums: this lane's kFindPer consecutive blocks and the
  // wave's inclusive scan of the lane sums (summed in block order)
  auto chunk = [&](int c0, double (&xs)[kFindPer], double& is) {
#pragma unroll
    for (int t = 0; t < kFindPer; ++t) {
      const int b = c0 + lane * kFindPer + t;
      xs[t] = b < nb ? ds[b].sw : 0.0;
    }
    double ls = 0.0;
#pragma unroll
    for (int t = 0; t < kFindPer; ++t) ls += xs[t];
    is = wave_incl_scan_f64(ls);
  };
  // the total, chunk totals summed in order (wave 0); the first chunk stays in registers
  double x[kFindPer], incl = 0.0;
  auto total = [&]() {
    chunk(0, x, incl);
    double s = readlane_d(incl, 63);
    for (int c0 = kChunk; c0 < nb; c0 += kChunk) {
      double y[kFindPer], iy;
      chunk(c0, y, iy);
      s += readlane_d(iy, 63);
    }
    if (lane == 0) s_tw = s;
  };
  // row A's record is requested before the block sums, so both arrive in one round trip
  const RowStats sa = a.stats[(size_t)i * (G + 1) + A];
  if (wave == 0) total();
  const DrawW dwt = draw_weights<LT>(a, i, cx, sa);
  // the request's banned tokens (checked by the row pass, which faults the
  // request on a bad list)
  int nban = 0;
  if (TOK && a.ban_off) {
    const int b0 = a.ban_off[i];
    nban = a.ban_off[i + 1] - b0;
    for (int t = tid; t < nban; t += kBlock) s_ban[t] = a.ban_ids[(size_t)b0 + t];
  }
  __syncthreads();
  // row A's penalty list (checked by the row pass likewise)
  int npen = 0;
  float theta = 1.f;
  if (TOK == 2) {
    Req rq;
    rq.id0 = rr.id0;
    npen = load_penalties(a, rq, i, A, (LDS_AS int*)s_pid, (LDS_AS float*)s_pd, (LDS_AS float*)s_stage, theta, false);
  }
  const Toks tk = toks((const LDS_AS int*)s_ban, nban, (const LDS_AS int*)s_pid, (const LDS_AS float*)s_pd,
                       (LDS_AS float*)s_stage + (threadIdx.x >> 6) * 512, npen, theta);
  // Weights of one lane's 8 tokens in block blk (512 tokens: step blk / 4,
  // wave range blk % 4) under draw mode md; lists applied token by token.
  auto block_weights = [&](int blk, int md, float w[8], int& base) -> bool {
    base = (blk / kWaves) * kStep + (blk % kWaves) * 512 + lane * kCh;
    LR lb = load_logits<LT, VEC>(lrow, base, V);
    F32::Raw qb = (md == 1) ? load_probs<VEC>(qrow, base, V) : F32::Raw{};
    if (TOK == 2 && tk.npen) {
      float dv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = tok_find(tk.pid, tk.npen, base + e);
        dv[e] = k >= 0 ? tk.pd[k] : __uint_as_float(0x7fffffffu);
      }
      pen_apply(lb, dv, tk.theta);
      if (md == 1) pen_apply_q(qb, dv);
    }
    if (TOK) {
      uint32_t m = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ban_has(tk.ban, tk.nban, base + e)) m |= 1u << e;
      if (m) {
        ban_logits(lb, m);
        ban_apply(qb, m, 0u);
      }
    }
    float lv[8], qv[8];
    LT::unpack(lb, lv);
    if (md == 1) F32::unpack(qb, qv);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = 0.f;
    DrawW dd = dwt;
    dd.mode = md;
    const bool prec = md == 1 && dd.temper && dd.dw.precise;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      w[e] = prec ? draw_weight<true>(lv[e], qv[e], base + e, dd) : draw_weight<false>(lv[e], qv[e], base + e, dd);
    return prec;
  };

  int dmode = mode;
  bool held = nb <= kChunk;  // wave 0 holds every block sum in registers
  if (!(s_tw > 0.0)) {
    // Zero residual (p' and q' agree and the draft token lies outside both
    // kept sets): the draw is from p'.  Rare: the block sums of p' are
    // formed here, by this workgroup alone.
    dmode = 0;
    held = false;
    for (int blk = wave; blk < nb; blk += kWaves) {
      float w[8];
      int base;
      block_weights(blk, 0, w, base);  // (mode 0: never the precise form)
      DrawSum d;
      d.sw = wave_sum_f64(lane_sum8(w));
      if (lane == 0) ds[blk] = d;
    }
    __syncthreads();
    if (wave == 0) total();
  }
  if (wave != 0) return;
  const double S = readlane_d(s_tw, 0);
  const double tau = (double)us * S;
  // the lane, then its block, where the running sum first exceeds tau; where
  // rounding leaves tau at or past the total, the last block of positive
  // weight, and there the last token of positive weight
  double pre = 0.0, pstar = 0.0;
  int bstar = -1, blast = -1;
  for (int c0 = 0; c0 < nb; c0 += kChunk) {
    if (!held) chunk(c0, x, incl);
    int lp = -1;
#pragma unroll
    for (int t = 0; t < kFindPer; ++t)
      if (x[t] > 0.0) lp = c0 + lane * kFindPer + t;
    blast = max(blast, wave_max_i(lp));
    if (bstar < 0) {
      const uint64_t hit = __ballot(lp >= 0 && pre + incl > tau);
      if (hit) {
        const int l = __ffsll((unsigned long long)hit) - 1;
        double run = pre + (l > 0 ? readlane_d(incl, l - 1) : 0.0);
        int bl = -1, blp = -1;
        double pb = 0.0, pbp = 0.0;
#pragma unroll
        for (int t = 0; t < kFindPer; ++t) {
          if (x[t] > 0.0) {
            if (bl < 0 && run + x[t] > tau) {
              bl = t;
              pb = run;
            }
            blp = t;
            pbp = run;
          }
          run += x[t];
        }
        if (bl < 0) {
          bl = blp;
          pb = pbp;
        }
        bstar = c0 + l * kFindPer + __builtin_amdgcn_readlane(bl, l);
        pstar = readlane_d(pb, l);
      } else {
        pre += readlane_d(incl, 63);
      }
    }
  }
  const bool last = bstar < 0;
  const int rstar = last ? blast : bstar;
  int z = -1;
  if (rstar >= 0) {
    float w[8];
    int base;
    const double ls = block_weights(rstar, dmode, w, base) ? lane_sum8_seq(w) : lane_sum8(w);
    double acc = pstar + (wave_incl_scan_f64(ls) - ls);
    int zz = INT_MAX, lastpos = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (w[e] > 0.f) lastpos = base + e;
      acc += (double)w[e];
      if (zz == INT_MAX && w[e] > 0.f && acc > tau) zz = base + e;
    }
    const int best = last ? INT_MAX : -wave_max_i(-zz);
    z = best != INT_MAX ? best : wave_max_i(lastpos);
  }
  if (lane == 0) {
    a.out_tokens[(size_t)i * (G + 1) + A] = z;
    if (a.d_resid) a.d_resid[i] = S;
  }
}

// One launch for the draw pass (calls without token lists and with kFinMinN
// to kFinMaxN requests): one kFinBlock-thread workgroup per request writes the
// outputs and, where row A made no draw of its own, forms the sum of the draw
// weights of each 512-token block of row A in LDS (wave w takes blocks w,
// w + kFinWaves, ..., kFinWin of them in flight), then searches them as the
// find kernel does.  Every block sum and the search stay in one workgroup:
// no hand-off between workgroups and no second launch.  The weights and lane
// sums are the draw kernel's (draw_w), so the block re-read for the token
// matches the sums.
template <class LT, bool VEC>
__global__ __launch_bounds__(kFinBlock) void finish_kernel(Args a) {
  typedef typename LT::Raw LR;
  extern __shared__ double s_fin[];  // [nb] block sums of row A
  __shared__ double s_tw;
  const int i = blockIdx.x;
  const DrawCtx<LT> cx = draw_ctx<LT>(a, i);
  const float us = a.u_sample[i];
  request_outputs(a, i, cx.rr, cx.A, cx.defer, cx.lanes, cx.lid, cx.ldr, cx.ldr64);
  if (!cx.defer) return;
  const int G = a.G, V = a.V, A = cx.A, mode = cx.mode;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const typename LT::T* lrow = cx.lrow;
  const float* qrow = cx.qrow;
  const int nb = cx.nsteps * kWaves;
  const DrawW dwt = draw_weights<LT>(a, i, cx, a.stats[(size_t)i * (G + 1) + A]);
  const bool precise = mode == 1 && dwt.temper && dwt.dw.precise;
  const bool filt = dwt.cut_p > -INFINITY || dwt.cut_q > -INFINITY;
  typedef std::integral_constant<int, 0> M0;
  typedef std::integral_constant<int, 1> M1;
  typedef std::integral_constant<int, 2> M2;
  typedef std::true_type Y;
  typedef std::false_type N;
  // Block sums of row A under the compile-time draw form (MODE, TEMPER, FILT,
  // PRECISE).  Blocks wholly inside the row: unconditional 16-byte loads, W
  // blocks of each wave in flight (a load that may fall back to element loads
  // puts a wait for every outstanding load at each of its branches).  The
  // row's partial last block, and every block without 16-byte loads or in the
  // precise form: one at a time through the element-wise path.
  const int nfull = VEC ? V / 512 : 0;
  auto sums = [&](auto md, auto tp, auto ft, auto pr) {
    constexpr int M = decltype(md)::value;
    constexpr bool P = decltype(pr)::value;
    auto weigh = [&](LR& l, F32::Raw& q, int b) -> double {
      const int base = b * 512 + lane * kCh;
      float lv[8], qv[8], w[8];
      LT::unpack(l, lv);
      if (M == 1) F32::unpack(q, qv);
      if constexpr (P) {
        double ls = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) ls += (double)draw_w<1, true, decltype(ft)::value, true>(lv[e], qv[e], base + e, dwt);
        return ls;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          w[e] = draw_w<M, decltype(tp)::value, decltype(ft)::value, false>(lv[e], M == 1 ? qv[e] : 0.f, base + e,
                                                                            dwt);
        return lane_sum8(w);
      }
    };
    int first = 0;  // the first block of the element-wise path
    if constexpr (VEC && !P) {
      first = nfull;
      for (int b0 = wave; b0 < nfull; b0 += kFinWaves * kFinWin) {
        LR l[kFinWin];
        F32::Raw q[kFinWin];
#pragma unroll
        for (int u = 0; u < kFinWin; ++u) {
          const int b = b0 + u * kFinWaves;
          const int base = (b < nfull ? b : b0) * 512 + lane * kCh;  // (past the last: b0 again, not used)
          l[u] = LT::load(lrow + base);
          if (M == 1) q[u] = F32::load(qrow + base);
        }
#pragma unroll
        for (int u = 0; u < kFinWin; ++u) {
          const int b = b0 + u * kFinWaves;
          if (b >= nfull) break;
          const double sw = wave_sum_f64(weigh(l[u], q[u], b));
          if (lane == 0) s_fin[b] = sw;
        }
      }
    }
    for (int b = first + wave; b < nb; b += kFinWaves) {
      const int base = b * 512 + lane * kCh;
      LR l = load_logits<LT, VEC>(lrow, base, V);
      F32::Raw q = M == 1 ? load_probs<VEC>(qrow, base, V) : F32::Raw{};
      const double sw = wave_sum_f64(weigh(l, q, b));
      if (lane == 0) s_fin[b] = sw;
    }
  };
  if (precise) {
    if (filt) sums(M1{}, Y{}, Y{}, Y{});
    else sums(M1{}, Y{}, N{}, Y{});
  } else if (mode == 1) {
    if (dwt.temper) {
      if (filt) sums(M1{}, Y{}, Y{}, N{});
      else sums(M1{}, Y{}, N{}, N{});
    } else {
      if (filt) sums(M1{}, N{}, Y{}, N{});
      else sums(M1{}, N{}, N{}, N{});
    }
  } else if (mode == 2) {
    if (filt) sums(M2{}, N{}, Y{}, N{});
    else sums(M2{}, N{}, N{}, N{});
  } else {
    if (filt) sums(M0{}, N{}, Y{}, N{});
    else sums(M0{}, N{}, N{}, N{});
  }
  __syncthreads();
  constexpr int kChunk = 64 * kFindPer;
  // one chunk of block sums: this lane's kFindPer consecutive blocks and the
  // wave's inclusive scan of the lane sums (summed in block order)
  auto chunk = [&](int c0, double (&xs)[kFindPer], double& is) {
#pragma unroll
    for (int t = 0; t < kFindPer; ++t) {
      const int b = c0 + lane * kFindPer + t;
      xs[t] = b < nb ? s_fin[b] : 0.0;
    }
    double ls = 0.0;
#pragma unroll
    for (int t = 0; t < kFindPer; ++t) ls += xs[t];
    is = wave_incl_scan_f64(ls);
  };
  double x[kFindPer], incl = 0.0;
  auto total = [&]() {
    chunk(0, x, incl);
    double s = readlane_d(incl, 63);
    for (int c0 = kChunk; c0 < nb; c0 += kChunk) {
      double y[kFindPer], iy;
      chunk(c0, y, iy);
      s += readlane_d(iy, 63);
    }
    if (lane == 0) s_tw = s;
  };
  if (wave == 0) total();
  __syncthreads();
  // weights of one lane's 8 tokens in block blk under draw mode md
  auto block_weights = [&](int blk, int md, float w[8], int& base) -> bool {
    base = blk * 512 + lane * kCh;
    LR lb = load_logits<LT, VEC>(lrow, base, V);
    F32::Raw qb = (md == 1) ? load_probs<VEC>(qrow, base, V) : F32::Raw{};
    float lv[8], qv[8];
    LT::unpack(lb, lv);
    if (md == 1) F32::unpack(qb, qv);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = 0.f;
    DrawW dd = dwt;
    dd.mode = md;
    const bool prec = md == 1 && dd.temper && dd.dw.precise;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      w[e] = prec ? draw_weight<true>(lv[e], qv[e], base + e, dd) : draw_weight<false>(lv[e], qv[e], base + e, dd);
    return prec;
  };
  int dmode = mode;
  bool held = nb <= kChunk;  // wave 0 holds every block sum in registers
  if (!(s_tw > 0.0)) {
    // Zero residual: the draw is from p'; its block sums replace the residual's.
    dmode = 0;
    held = false;
    if (filt) sums(M0{}, N{}, Y{}, N{});
    else sums(M0{}, N{}, N{}, N{});
    __syncthreads();
    if (wave == 0) total();
  }
  if (wave != 0) return;
  const double S = readlane_d(s_tw, 0);
  const double tau = (double)us * S;
  double pre = 0.0, pstar = 0.0;
  int bstar = -1, blast = -1;
  for (int c0 = 0; c0 < nb; c0 += kChunk) {
    if (!held) chunk(c0, x, incl);
    int lp = -1;
#pragma unroll
    for (int t = 0; t < kFindPer; ++t)
      if (x[t] > 0.0) lp = c0 + lane * kFindPer + t;
    blast = max(blast, wave_max_i(lp));
    if (bstar < 0) {
      const uint64_t hit = __ballot(lp >= 0 && pre + incl > tau);
      if (hit) {
        const int l = __ffsll((unsigned long long)hit) - 1;
        double run = pre + (l > 0 ? readlane_d(incl, l - 1) : 0.0);
        int bl = -1, blp = -1;
        double pb = 0.0, pbp = 0.0;
#pragma unroll
        for (int t = 0; t < kFindPer; ++t) {
          if (x[t] > 0.0) {
            if (bl < 0 && run + x[t] > tau) {
              bl = t;
              pb = run;
            }
            blp = t;
            pbp = run;
          }
          run += x[t];
        }
        if (bl < 0) {
          bl = blp;
          pb = pbp;
        }
        bstar = c0 + l * kFindPer + __builtin_amdgcn_readlane(bl, l);
        pstar = readlane_d(pb, l);
      } else {
        pre += readlane_d(incl, 63);
      }
    }
  }
  const bool last = bstar < 0;
  const int rstar = last ? blast : bstar;
  int z = -1;
  if (rstar >= 0) {
    float w[8];
    int base;
    const double ls = block_weights(rstar, dmode, w, base) ? lane_sum8_seq(w) : lane_sum8(w);
    double acc = pstar + (wave_incl_scan_f64(ls) - ls);
    int zz = INT_MAX, lastpos = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (w[e] > 0.f) lastpos = base + e;
      acc += (double)w[e];
      if (zz == INT_MAX && w[e] > 0.f && acc > tau) zz = base + e;
    }
    const int best = last ? INT_MAX : -wave_max_i(-zz);
    z = best != INT_MAX ? best : wave_max_i(lastpos);
  }
  if (lane == 0) {
    a.out_tokens[(size_t)i * (G + 1) + A] = z;
    if (a.d_resid) a.d_resid[i] = S;
  }
}

// ------------------------------------------------------------------------------------------
// KV bookkeeping after a verify call
// ------------------------------------------------------------------------------------------

struct RollbackArgs {
  int N, G;
  const int32_t* cu;         // [N] flattened layout, or nullptr
  const int32_t* ids;        // [N, G] padded layout (gamma_i = first negative id), or nullptr
  const int32_t* num_accepted;
  int32_t* num_computed;     // [N] or nullptr
  int32_t* num_placeholders; // [N] or nullptr
  int32_t* slots;            // aligned with the drafts ([T] or [N, G]), or nullptr
};

// One thread per request (KV page "投机解码如何与 KV Cache 交互", sections
// 3.1 and 3.2; vLLM page, the padded drafter batch paragraph): the gamma_i - A_i
// rejected drafts are taken back from num_computed_tokens and from the
// placeholder count when those are positive, and their KV slots become
// PADDING_SLOT_ID (-1).  A request with A_i outside [0, gamma_i] (a faulted
// verify) or an invalid count is left as it is.
__global__ __launch_bounds__(kBlock) void rollback_kernel(RollbackArgs r) {
  const int i = (int)(blockIdx.x * kBlock + threadIdx.x);
  if (i >= r.N) return;
  int gamma, id0;
  if (r.cu) {
    const int prev = i ? r.cu[i - 1] : 0;
    gamma = r.cu[i] - prev;
    id0 = prev;
  } else {
    gamma = r.G;
    for (int jj = r.G - 1; jj >= 0; --jj)
      if (r.ids[(size_t)i * r.G + jj] < 0) gamma = jj;
    id0 = i * r.G;
  }
  const int A = r.num_accepted[i];
  if (A < 0 || A > gamma || gamma > r.G) return;
  const int rejected = gamma - A;
  if (r.num_computed && r.num_computed[i] > 0) r.num_computed[i] -= rejected;
  if (r.num_placeholders && r.num_placeholders[i] > 0) r.num_placeholders[i] -= rejected;
  if (r.slots)
    for (int j = A; j < gamma; ++j) r.slots[(size_t)id0 + j] = -1;
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// the workspace starts with this call's fault count (one 256-byte block)
constexpr size_t kHeadBytes = 256;
size_t stats_bytes(int N, int G) { return align_up((size_t)N * (G + 1) * sizeof(RowStats), 256); }
size_t rec_bytes(int N) { return align_up((size_t)N * sizeof(ReqRec), 256); }
size_t plan_bytes(int N, int G) { return align_up(((size_t)N * G + 1) * sizeof(int), 256); }
size_t dsum_bytes(int N, int V) {
  return align_up((size_t)N * ((V + kStep - 1) / kStep) * kWaves * sizeof(DrawSum), 256);
}
size_t draw_parts(int V) { return ((size_t)(V + kStep - 1) / kStep + kDrawSpan - 1) / kDrawSpan; }

struct Events {
  hipEvent_t start, mid, end;
};

template <class LT, bool VEC, int TOK>
hipError_t launch(const Args& a, hipStream_t stream, const Events& ev) {
  const long rows = row_blocks(a.N, a.G, a.synthetic, a.direct);
  hipError_t e;
  if (!a.direct) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kBlock), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the row pass's events travel in its own dispatch (start and end of the
  // kernel), so timing it adds no packets before or after it on the stream
  if (ev.start || ev.mid)
    hipExtLaunchKernelGGL((row_kernel<LT, VEC, TOK>), dim3((unsigned)rows), dim3(kBlock), 0, stream, ev.start, ev.mid,
                          0u, a);
  else
    hipLaunchKernelGGL((row_kernel<LT, VEC, TOK>), dim3((unsigned)rows), dim3(kBlock), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the draw pass: one fused launch for calls without token lists and with
  // kFinMinN to kFinMaxN requests (row A's block sums in LDS, at most 48 KB of
  // them: V up to 3,145,728); otherwise block sums over many workgroups, then the search.  The
  // fused launch saves a launch, but gives each request's draw to one
  // workgroup: with fewer requests it leaves CUs idle, with more it loads
  // some CUs with two deferred rows and others with one.
  const size_t fin_lds = (size_t)((a.V + kStep - 1) / kStep) * kWaves * sizeof(double);
  if (TOK == 0 && a.N >= kFinMinN && a.N <= kFinMaxN && fin_lds <= 48 * 1024) {
    hipLaunchKernelGGL((finish_kernel<LT, VEC>), dim3((unsigned)a.N), dim3(kFinBlock), fin_lds, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((draw_kernel<LT, VEC, TOK>), dim3((unsigned)((long)a.N * a.dparts)), dim3(kBlock), 0, stream,
                       a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((find_kernel<LT, VEC, TOK>), dim3((unsigned)a.N), dim3(kBlock), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev.end && (e = hipEventRecord(ev.end, stream)) != hipSuccess) return e;
  return hipSuccess;
}

// Where the drafts sit: the padded layout (cu == nullptr) or the flattened one.
struct Layout {
  const int32_t* cu;
  const uint8_t* has_q;
  int T;
};

// Penalty lists per position and the per-request penalties (all nullptr: none).
struct Penalties {
  const int32_t *off, *ids, *cnt;
  const float *rep, *pres, *freq;
};

int run(int N, int G, int V, const Layout& lay, bool synthetic, const float* srates, const int32_t* ban_off,
        const int32_t* ban_ids, const Penalties& pen, const int32_t* tidx, const int32_t* bidx, int R, const int32_t* ids, const float* q, const void* logits, int dtype,
        const float* temperature, const int32_t* top_k, const float* top_p, const float* u_accept,
        const float* u_sample, int32_t* out_tokens, int32_t* out_num, double* p_y, double* q_y, double* resid,
        int32_t* fault, void* workspace, size_t workspace_bytes, void* stream, const Events& ev) {
  if (N < 0 || G < 0 || G > kMaxGamma || V < 1) return SPEC_VERIFY_ERR_SHAPE;
  const bool flat = lay.cu != nullptr;
  if (flat && (lay.T < 0 || (long long)lay.T > (long long)N * G)) return SPEC_VERIFY_ERR_SHAPE;
  if (dtype != SPEC_VERIFY_F32 && dtype != SPEC_VERIFY_BF16) return SPEC_VERIFY_ERR_DTYPE;
  if ((long long)V * (G + 1) > (1LL << 40) || V > 0x7fffffff - 2 * kStep) return SPEC_VERIFY_ERR_SHAPE;
  // a dispatch holds its grid size in work-items as a 32-bit number
  const long long dparts = (long long)draw_parts(V);
  if ((long long)row_blocks(N, G, synthetic, !lay.cu && !synthetic) * kBlock > 0xffffffffLL ||
      (long long)N * dparts * kBlock > 0xffffffffLL)
    return SPEC_VERIFY_ERR_SHAPE;
  if (N == 0) return SPEC_VERIFY_OK;
  if (!logits || !u_sample || !out_tokens || !out_num) return SPEC_VERIFY_ERR_NULL;
  if ((flat ? lay.T : G) > 0 && (!ids || !u_accept)) return SPEC_VERIFY_ERR_NULL;
  const size_t need = spec_verify_workspace_size(N, G, V);
  if (!workspace) return SPEC_VERIFY_ERR_NULL;
  if (workspace_bytes < need) return SPEC_VERIFY_ERR_WORKSPACE;

  Args a;
  a.N = N;
  a.G = G;
  a.V = V;
  a.ids = ids;
  a.q = q;
  a.logits = logits;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.u_accept = u_accept;
  a.u_sample = u_sample;
  a.out_tokens = out_tokens;
  a.out_num = out_num;
  a.d_py = p_y;
  a.d_qy = q_y;
  a.d_resid = resid;
  a.d_fault = fault;
  char* ws = reinterpret_cast<char*>(workspace);
  a.nfault = reinterpret_cast<unsigned int*>(ws);
  a.stats = reinterpret_cast<RowStats*>(ws + kHeadBytes);
  size_t off = kHeadBytes + stats_bytes(N, G);
  a.rec = reinterpret_cast<ReqRec*>(ws + off);
  off += rec_bytes(N);
  a.dsum = reinterpret_cast<DrawSum*>(ws + off);
  off += dsum_bytes(N, V);
  a.plan = reinterpret_cast<int*>(ws + off);
  a.dparts = (int)dparts;
  a.cu = lay.cu;
  a.has_q = lay.has_q;
  a.T = lay.T;
  a.tidx = tidx;
  a.bidx = bidx;
  a.R = R;
  a.ban_off = ban_off;
  a.ban_ids = ban_ids;
  a.pen_off = pen.off;
  a.pen_ids = pen.ids;
  a.pen_cnt = pen.cnt;
  a.pen_rep = pen.rep;
  a.pen_pres = pen.pres;
  a.pen_freq = pen.freq;
  a.synthetic = synthetic ? 1 : 0;
  a.direct = (!lay.cu && !synthetic) ? 1 : 0;
  a.dslots = direct_slots(G);
  a.srates = srates;

  // 16-byte vector loads need every row start aligned: V a multiple of 8 and
  // 16-byte aligned base pointers
  const bool vec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0) && (!q || (uintptr_t)q % 16 == 0);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (pen.off) {
    if (dtype == SPEC_VERIFY_BF16)
      e = vec ? launch<Bf16, true, 2>(a, s, ev) : launch<Bf16, false, 2>(a, s, ev);
    else
      e = vec ? launch<F32, true, 2>(a, s, ev) : launch<F32, false, 2>(a, s, ev);
  } else if (ban_off) {
    if (dtype == SPEC_VERIFY_BF16)
      e = vec ? launch<Bf16, true, 1>(a, s, ev) : launch<Bf16, false, 1>(a, s, ev);
    else
      e = vec ? launch<F32, true, 1>(a, s, ev) : launch<F32, false, 1>(a, s, ev);
  } else {
    if (dtype == SPEC_VERIFY_BF16)
      e = vec ? launch<Bf16, true, 0>(a, s, ev) : launch<Bf16, false, 0>(a, s, ev);
    else
      e = vec ? launch<F32, true, 0>(a, s, ev) : launch<F32, false, 0>(a, s, ev);
  }
  return e == hipSuccess ? SPEC_VERIFY_OK : SPEC_VERIFY_ERR_HIP;
}

// ------------------------------------------------------------------------------------------
// the entry point that allocates nothing: a file-scope scratch array as its workspace
// ------------------------------------------------------------------------------------------

// Every GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only the
// address hipGetSymbolAddress returns for the current device is ever passed to
// a kernel.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, set on first use

// The current device's address of `scratch` (looked up once per device, with
// that device current).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_VERIFY_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_VERIFY_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_VERIFY_OK;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int N, int gmax, int V) {
  if (N <= 0 || gmax < 0 || V <= 0) return 256;
  return kHeadBytes + stats_bytes(N, gmax) + rec_bytes(N) + dsum_bytes(N, V) + plan_bytes(N, gmax);
}

int spec_verify(int N, int gmax, int V, const int32_t* draft_ids, const float* draft_probs, const void* target_logits,
                int logits_dtype, const float* temperature, const int32_t* top_k, const float* top_p,
                const float* u_accept, const float* u_sample, int32_t* out_tokens, int32_t* out_num_accepted,
                void* workspace, size_t workspace_bytes, void* stream) {
  return run(N, gmax, V, Layout{nullptr, nullptr, 0}, false, nullptr, nullptr, nullptr, Penalties{}, nullptr, nullptr, 0, draft_ids, draft_probs, target_logits, logits_dtype, temperature, top_k, top_p, u_accept,
             u_sample, out_tokens, out_num_accepted, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes,
             stream, Events{nullptr, nullptr, nullptr});
}

int spec_verify_diag(int N, int gmax, int V, const int32_t* draft_ids, const float* draft_probs,
                     const void* target_logits, int logits_dtype, const float* temperature, const int32_t* top_k,
                     const float* top_p, const float* u_accept, const float* u_sample, int32_t* out_tokens,
                     int32_t* out_num_accepted, double* p_y, double* q_y, double* resid_mass, int32_t* fault,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return run(N, gmax, V, Layout{nullptr, nullptr, 0}, false, nullptr, nullptr, nullptr, Penalties{}, nullptr, nullptr, 0, draft_ids, draft_probs, target_logits, logits_dtype, temperature, top_k, top_p, u_accept,
             u_sample, out_tokens, out_num_accepted, p_y, q_y, resid_mass, fault, workspace, workspace_bytes, stream,
             Events{nullptr, nullptr, nullptr});
}

int spec_verify_timed(int N, int gmax, int V, const int32_t* draft_ids, const float* draft_probs,
                      const void* target_logits, int logits_dtype, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* u_accept, const float* u_sample, int32_t* out_tokens,
                      int32_t* out_num_accepted, double* p_y, double* q_y, double* resid_mass, int32_t* fault,
                      void* workspace, size_t workspace_bytes, void* stream, void* ev_start, void* ev_mid,
                      void* ev_end) {
  return run(N, gmax, V, Layout{nullptr, nullptr, 0}, false, nullptr, nullptr, nullptr, Penalties{}, nullptr, nullptr, 0, draft_ids, draft_probs, target_logits, logits_dtype, temperature, top_k, top_p, u_accept,
             u_sample, out_tokens, out_num_accepted, p_y, q_y, resid_mass, fault, workspace, workspace_bytes, stream,
             Events{reinterpret_cast<hipEvent_t>(ev_start), reinterpret_cast<hipEvent_t>(ev_mid),
                    reinterpret_cast<hipEvent_t>(ev_end)});
}

int spec_verify_flat(int N, int gmax, int V, int num_drafts, const int32_t* cu_num_draft_tokens,
                     const int32_t* draft_ids, const float* draft_probs, const uint8_t* has_draft_probs,
                     const void* target_logits, int logits_dtype, const float* temperature, const int32_t* top_k,
                     const float* top_p, const float* u_accept, const float* u_sample, int32_t* out_tokens,
                     int32_t* out_num_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  if (N > 0 && !cu_num_draft_tokens) return SPEC_VERIFY_ERR_NULL;
  return run(N, gmax, V, Layout{cu_num_draft_tokens, has_draft_probs, num_drafts}, false, nullptr, nullptr, nullptr, Penalties{}, nullptr, nullptr, 0, draft_ids, draft_probs,
             target_logits, logits_dtype, temperature, top_k, top_p, u_accept, u_sample, out_tokens,
             out_num_accepted, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream,
             Events{nullptr, nullptr, nullptr});
}

int spec_verify_flat_timed(int N, int gmax, int V, int num_drafts, const int32_t* cu_num_draft_tokens,
                           const int32_t* draft_ids, const float* draft_probs, const uint8_t* has_draft_probs,
                           const void* target_logits, int logits_dtype, const float* temperature,
                           const int32_t* top_k, const float* top_p, const float* u_accept, const float* u_sample,
                           int32_t* out_tokens, int32_t* out_num_accepted, double* p_y, double* q_y,
                           double* resid_mass, int32_t* fault, void* workspace, size_t workspace_bytes, void* stream,
                           void* ev_start, void* ev_mid, void* ev_end) {
  if (N > 0 && !cu_num_draft_tokens) return SPEC_VERIFY_ERR_NULL;
  return run(N, gmax, V, Layout{cu_num_draft_tokens, has_draft_probs, num_drafts}, false, nullptr, nullptr, nullptr, Penalties{}, nullptr, nullptr, 0, draft_ids, draft_probs,
             target_logits, logits_dtype, temperature, top_k, top_p, u_accept, u_sample, out_tokens,
             out_num_accepted, p_y, q_y, resid_mass, fault, workspace, workspace_bytes, stream,
             Events{reinterpret_cast<hipEvent_t>(ev_start), reinterpret_cast<hipEvent_t>(ev_mid),
                    reinterpret_cast<hipEvent_t>(ev_end)});
}

int spec_verify_flat_ex(int N, int gmax, int V, int num_drafts, const int32_t* cu_num_draft_tokens,
                        const int32_t* draft_ids, const float* draft_probs, const uint8_t* has_draft_probs,
                        const void* target_logits, int logits_rows, const int32_t* target_logits_indices,
                        const int32_t* bonus_logits_indices, int logits_dtype, const float* temperature,
                        const int32_t* top_k, const float* top_p, const int32_t* banned_offsets,
                        const int32_t* banned_ids, const int32_t* penalty_offsets, const int32_t* penalty_ids,
                        const int32_t* penalty_counts, const float* repetition_penalty, const float* presence_penalty,
                        const float* frequency_penalty, const float* u_accept, const float* u_sample,
                        int32_t* out_tokens, int32_t* out_num_accepted, double* p_y, double* q_y, double* resid_mass,
                        int32_t* fault, void* workspace, size_t workspace_bytes, void* stream, void* ev_start,
                        void* ev_mid, void* ev_end) {
  if (N > 0 && !cu_num_draft_tokens) return SPEC_VERIFY_ERR_NULL;
  // the bonus indices and the offsets select the options; their companions
  // may be NULL only where nothing would be read through them
  if (N > 0 && target_logits_indices && !bonus_logits_indices) return SPEC_VERIFY_ERR_NULL;
  if (N > 0 && num_drafts > 0 && bonus_logits_indices && !target_logits_indices) return SPEC_VERIFY_ERR_NULL;
  if (N > 0 && banned_ids && !banned_offsets) return SPEC_VERIFY_ERR_NULL;
  if (N > 0 && !penalty_offsets && (penalty_ids || penalty_counts || repetition_penalty || presence_penalty ||
                                    frequency_penalty))
    return SPEC_VERIFY_ERR_NULL;
  if (N > 0 && penalty_offsets && (penalty_ids != nullptr) != (penalty_counts != nullptr)) return SPEC_VERIFY_ERR_NULL;
  if (N > 0 && (logits_rows < 1 || (!bonus_logits_indices && (long long)logits_rows < (long long)num_drafts + N)))
    return SPEC_VERIFY_ERR_SHAPE;
  const Penalties pen{penalty_offsets, penalty_ids, penalty_counts, repetition_penalty, presence_penalty,
                      frequency_penalty};
  return run(N, gmax, V, Layout{cu_num_draft_tokens, has_draft_probs, num_drafts}, false, nullptr, banned_offsets,
             banned_ids, pen, target_logits_indices, bonus_logits_indices, logits_rows, draft_ids, draft_probs,
             target_logits, logits_dtype, temperature, top_k, top_p, u_accept, u_sample, out_tokens, out_num_accepted,
             p_y, q_y, resid_mass, fault, workspace, workspace_bytes, stream,
             Events{reinterpret_cast<hipEvent_t>(ev_start), reinterpret_cast<hipEvent_t>(ev_mid),
                    reinterpret_cast<hipEvent_t>(ev_end)});
}

int spec_verify_flat_synthetic(int N, int gmax, int V, int num_drafts, const int32_t* cu_num_draft_tokens,
                               const int32_t* draft_ids, const float* draft_probs, const uint8_t* has_draft_probs,
                               const void* target_logits, int logits_dtype, const float* temperature,
                               const int32_t* top_k, const float* top_p, const float* synthetic_rates,
                               const float* u_accept, const float* u_sample, int32_t* out_tokens,
                               int32_t* out_num_accepted, int32_t* fault, void* workspace, size_t workspace_bytes,
                               void* stream, void* ev_start, void* ev_mid, void* ev_end) {
  if (N > 0 && !cu_num_draft_tokens) return SPEC_VERIFY_ERR_NULL;
  if (N > 0 && gmax > 0 && !synthetic_rates) return SPEC_VERIFY_ERR_NULL;
  return run(N, gmax, V, Layout{cu_num_draft_tokens, has_draft_probs, num_drafts}, true, synthetic_rates, nullptr, nullptr, Penalties{}, nullptr, nullptr, 0, draft_ids, draft_probs, target_logits, logits_dtype,
             temperature, top_k, top_p, u_accept, u_sample, out_tokens, out_num_accepted, nullptr, nullptr, nullptr,
             fault, workspace, workspace_bytes, stream,
             Events{reinterpret_cast<hipEvent_t>(ev_start), reinterpret_cast<hipEvent_t>(ev_mid),
                    reinterpret_cast<hipEvent_t>(ev_end)});
}

int spec_verify_rollback(int N, int gmax, const int32_t* cu_num_draft_tokens, const int32_t* draft_ids,
                         const int32_t* num_accepted, int32_t* num_computed_tokens, int32_t* num_output_placeholders,
                         int32_t* slot_mapping, void* stream) {
  if (N < 0 || gmax < 0 || gmax > kMaxGamma) return SPEC_VERIFY_ERR_SHAPE;
  if (N == 0) return SPEC_VERIFY_OK;
  if (!num_accepted) return SPEC_VERIFY_ERR_NULL;
  if ((cu_num_draft_tokens != nullptr) == (draft_ids != nullptr) && gmax > 0) return SPEC_VERIFY_ERR_NULL;
  RollbackArgs r;
  r.N = N;
  r.G = gmax;
  r.cu = cu_num_draft_tokens;
  r.ids = cu_num_draft_tokens ? nullptr : draft_ids;
  r.num_accepted = num_accepted;
  r.num_computed = num_computed_tokens;
  r.num_placeholders = num_output_placeholders;
  r.slots = slot_mapping;
  hipLaunchKernelGGL(rollback_kernel, dim3((unsigned)((N + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                     reinterpret_cast<hipStream_t>(stream), r);
  return hipGetLastError() == hipSuccess ? SPEC_VERIFY_OK : SPEC_VERIFY_ERR_HIP;
}

int spec_verify_static(int N, int gmax, int V, const int32_t* draft_ids, const float* draft_probs,
                       const void* target_logits, int logits_dtype, const float* temperature, const int32_t* top_k,
                       const float* top_p, const float* u_accept, const float* u_sample, int32_t* out_tokens,
                       int32_t* out_num_accepted, void* stream) {
  // the size checks come first, so that a refused call touches no device state
  if (N < 0 || gmax < 0 || gmax > kMaxGamma || V < 1) return SPEC_VERIFY_ERR_SHAPE;
  if (N == 0) return SPEC_VERIFY_OK;
  if (spec_verify_workspace_size(N, gmax, V) > kStaticScratchBytes) return SPEC_VERIFY_ERR_SCRATCH;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != SPEC_VERIFY_OK) return rc;
  return spec_verify(N, gmax, V, draft_ids, draft_probs, target_logits, logits_dtype, temperature, top_k, top_p,
                     u_accept, u_sample, out_tokens, out_num_accepted, ws, kStaticScratchBytes, stream);
}

size_t spec_verify_static_scratch_bytes(void) { return kStaticScratchBytes; }

int spec_verify_device_errors(const void* workspace, size_t workspace_bytes, void* stream, int32_t* count) {
  if (!workspace || !count) return SPEC_VERIFY_ERR_NULL;
  if (workspace_bytes < kHeadBytes) return SPEC_VERIFY_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned int n = 0u;
  if (hipMemcpyAsync(&n, workspace, sizeof(n), hipMemcpyDeviceToHost, s) != hipSuccess) return SPEC_VERIFY_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SPEC_VERIFY_ERR_HIP;
  *count = (int32_t)n;
  return SPEC_VERIFY_OK;
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SPEC_VERIFY_OK: return "ok";
    case SPEC_VERIFY_ERR_NULL: return "a required pointer is NULL";
    case SPEC_VERIFY_ERR_SHAPE: return "N, gmax or V out of range";
    case SPEC_VERIFY_ERR_DTYPE: return "unknown logits dtype";
    case SPEC_VERIFY_ERR_WORKSPACE: return "workspace smaller than spec_verify_workspace_size";
    case SPEC_VERIFY_ERR_HIP: return "HIP runtime error";
    case SPEC_VERIFY_ERR_SCRATCH: return "workspace for these sizes exceeds the static scratch of spec_verify_static";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return 1; }

}  // extern "C"
