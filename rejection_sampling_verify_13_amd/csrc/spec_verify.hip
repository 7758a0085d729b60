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
// Two kernels per call, both on the caller's stream:
//   row_kernel    one 256-thread workgroup per (request, position) row.  It
//                 streams the target-logit row and, at draft positions of
//                 sampled requests, the draft-probability row once with 16-byte
//                 nontemporal loads, and reduces: row max, sum of exp over the
//                 row (fp32 terms, fp64 accumulation), sum of q^(1/T), draft-row
//                 validity, greedy argmax.  With top-k active (k <= kKFast) each
//                 wave keeps an LDS candidate buffer behind a rising threshold
//                 that never exceeds the true k-th largest value, so one pass
//                 yields the kept set; other filter settings use a radix select
//                 that re-reads the row.  p'(y) and q'(y) are evaluated in fp64
//                 and the acceptance flag u * q'(y) < p'(y) is stored.
//   finish_kernel one workgroup per request: ballot over the acceptance flags
//                 gives the first rejection A; greedy requests take the stored
//                 argmax, sampled ones draw by inverse CDF over ascending token
//                 id, either from the stored kept list of row A (filters active)
//                 or by two passes over row A (chunk sums, then the crossing
//                 chunk).  Outputs are written in the -1 padded layout.
//
// Compile: hipcc --offload-arch=gfx950 -O3 -shared -fPIC
//          -Xclang -target-feature -Xclang -packed-fp32-ops

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "spec_verify.h"

namespace {

constexpr int kBlock = 256;             // threads per workgroup (4 waves)
constexpr int kWaves = kBlock / 64;
constexpr int kCh = 8;                  // tokens per thread per step
constexpr int kStep = kBlock * kCh;     // tokens per workgroup step (2048)
constexpr int kWcap = 384;              // candidate slots per wave and distribution
constexpr int kKFast = 128;             // largest top_k served by the candidate buffers
constexpr int kListMax = 512;           // merged kept-set capacity (LDS)
constexpr int kLcap = kListMax;         // kept-list entries stored per row
constexpr int kMaxChunks = 512;         // chunk sums held by the draw
constexpr int kMaxGamma = 64;
constexpr float kLog2e = 1.4426950408889634f;

enum {
  kFaultDraftId = SPEC_VERIFY_FAULT_DRAFT_ID,
  kFaultTemperature = SPEC_VERIFY_FAULT_TEMPERATURE,
  kFaultTopP = SPEC_VERIFY_FAULT_TOP_P,
  kFaultTargetRow = SPEC_VERIFY_FAULT_TARGET_ROW,
  kFaultDraftRow = SPEC_VERIFY_FAULT_DRAFT_ROW,
  kFaultDraftMass = SPEC_VERIFY_FAULT_DRAFT_MASS,
};

// Per-row results of row_kernel (64 bytes).
struct RowStats {
  float m;        // max logit of the row
  float cut_p;    // target token kept iff logit >= cut_p
  float cut_q;    // draft token kept iff q >= cut_q
  int argmax;     // greedy rows: lowest id of the max logit
  double z;       // sum over the kept set of exp((l - m) / T)
  double r;       // sum over the kept set of q^(1/T)
  double p_y;     // p'(y) at a draft position
  double q_y;     // q'(y) at a draft position
  int flags;      // bit 0: accepted; bits 8..15: fault bits
  int nlist;      // entries of the stored kept list (-1: none stored)
  int pad[2];
};
static_assert(sizeof(RowStats) == 64, "RowStats layout");

struct ListEntry {
  int id;
  float val;      // the logit
  double e;       // exp((l - m) / T)
};

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
  ListEntry* lists;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// element access
// ------------------------------------------------------------------------------------------

struct Bf16 {
  typedef uint16_t T;
  static constexpr int kKeyBits = 16;
  __device__ static float at(const uint16_t* p, size_t x) { return __uint_as_float((uint32_t)p[x] << 16); }
  __device__ static void load8(const uint16_t* p, float v[8]) {
    u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xffff0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xffff0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

struct F32 {
  typedef float T;
  static constexpr int kKeyBits = 32;
  __device__ static float at(const float* p, size_t x) { return p[x]; }
  __device__ static void load8(const float* p, float v[8]) {
    u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
};

// Logits of one step: 8 consecutive tokens from `base`; positions at or past V
// read as -inf (no mass, never kept by a finite threshold, never an argmax).
template <class LT, bool VEC>
__device__ inline void load_logits(const typename LT::T* row, int base, int V, float v[8]) {
  if (VEC) {
    if (base < V) {
      LT::load8(row + base, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (base + e < V) ? LT::at(row, (size_t)(base + e)) : -INFINITY;
  }
}

// Draft probabilities of one step; positions at or past V read as 0.
template <bool VEC>
__device__ inline void load_q(const float* row, int base, int V, float v[8]) {
  if (VEC) {
    if (base < V) {
      F32::load8(row + base, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (base + e < V) ? row[base + e] : 0.f;
  }
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

__device__ inline float max8(const float v[8]) {
  float a = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
  float b = __builtin_fmaxf(__builtin_fmaxf(v[4], v[5]), __builtin_fmaxf(v[6], v[7]));
  return __builtin_fmaxf(a, b);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// q^(1/T) in fp64, the same expression wherever a single value is needed
__device__ inline double temper_q(float q, float T) {
  return T == 1.f ? (double)q : pow((double)q, 1.0 / (double)T);
}

// ------------------------------------------------------------------------------------------
// wave / block helpers
// ------------------------------------------------------------------------------------------

__device__ inline int lane_id() { return threadIdx.x & 63; }
__device__ inline uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

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
__device__ inline float wave_min_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline uint32_t wave_max_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
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
__device__ inline int wave_or_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o);
  return v;
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
__device__ inline float block_min_f(float v, float* red) {
  v = wave_min_f(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = __builtin_fminf(__builtin_fminf(red[0], red[1]), __builtin_fminf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ inline uint32_t block_max_u(uint32_t v, uint32_t* red) {
  v = wave_max_u(v);
  if (lane_id() == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = max(max(red[0], red[1]), max(red[2], red[3]));
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

// Exclusive prefix sum over the block in thread order (fp64); *total gets the sum.
__device__ inline double block_exscan_d(double v, double* red, double* total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) red[w] = inc;
  __syncthreads();
  double before = 0.0;
  for (int k = 0; k < w; ++k) before += red[k];
  *total = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return before + inc - v;
}

// ------------------------------------------------------------------------------------------
// request parameters
// ------------------------------------------------------------------------------------------

struct Req {
  int gamma;      // number of draft tokens
  float T;        // temperature
  int k;          // top_k (raw)
  float p;        // top_p (raw)
  int fault;      // parameter faults
  bool greedy;
  bool kact;      // top-k filter active
  bool pact;      // top-p filter active
};

// Every wave of the block evaluates this redundantly (gmax <= 64 ids).
__device__ inline Req load_req(const Args& a, int i) {
  Req r;
  const int lane = lane_id();
  const int32_t* ids = a.ids + (size_t)i * a.G;
  int id = (lane < a.G) ? ids[lane] : -1;
  uint64_t neg = __ballot(lane < a.G && id < 0);
  r.gamma = neg ? (__ffsll((unsigned long long)neg) - 1) : a.G;
  uint64_t bad = __ballot(lane < r.gamma && id >= a.V);
  r.fault = bad ? kFaultDraftId : 0;
  r.T = a.temperature ? a.temperature[i] : 1.f;
  r.k = a.top_k ? a.top_k[i] : 0;
  r.p = a.top_p ? a.top_p[i] : 1.f;
  const float T = r.T;
  if (isnan(T) || T < 0.f || isinf(T) || (T > 0.f && T < FLT_MIN)) r.fault |= kFaultTemperature;
  r.greedy = (T == 0.f);
  if (!r.greedy && !(r.fault & kFaultTemperature) && (isnan(r.p) || r.p <= 0.f)) r.fault |= kFaultTopP;
  r.kact = r.k >= 1 && r.k < a.V;
  r.pact = r.p < 1.f;
  return r;
}

// ------------------------------------------------------------------------------------------
// candidate buffers (top-k by rising threshold)
// ------------------------------------------------------------------------------------------

struct Cand {
  float* val;     // this wave's slots in LDS
  int* id;
  int cnt;        // wave-uniform
  float thr;      // wave-uniform: never above the k-th largest value seen
  bool overflow;  // wave-uniform: too many ties to stay within the slots
};

// Key of the k-th largest entry (by okey) over up to four LDS segments
// vals[s * stride .. + cnt[s]).  Requires 1 <= k <= total entries.  All 64
// lanes of the calling wave must be active.
__device__ uint32_t wave_kth_key(const float* vals, int stride, const int cnt[4], int nseg, int k, int key_bits,
                                 uint32_t* hist) {
  const int lane = lane_id();
  uint32_t prefix = 0, above = 0;
  for (int shift = 24; shift >= 32 - key_bits; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hist[b] = 0u;
    wave_lds_sync();
    const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
    for (int s = 0; s < nseg; ++s) {
      for (int e = lane; e < cnt[s]; e += 64) {
        uint32_t key = okey(vals[s * stride + e]);
        if ((key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
    }
    wave_lds_sync();
    uint32_t h0 = hist[lane * 4], h1 = hist[lane * 4 + 1], h2 = hist[lane * 4 + 2], h3 = hist[lane * 4 + 3];
    uint32_t local = h0 + h1 + h2 + h3, suf = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t t = (uint32_t)__shfl_down((int)suf, o);
      if (lane + o < 64) suf += t;
    }
    uint64_t okm = __ballot(above + suf >= (uint32_t)k);
    const int L = 63 - __clzll((long long)okm);
    uint32_t cum = (uint32_t)__shfl((int)(above + suf - local), L);
    uint32_t b3 = (uint32_t)__shfl((int)h3, L), b2 = (uint32_t)__shfl((int)h2, L), b1 = (uint32_t)__shfl((int)h1, L);
    int d;
    if (cum + b3 >= (uint32_t)k) {
      d = 3;
    } else {
      cum += b3;
      if (cum + b2 >= (uint32_t)k) {
        d = 2;
      } else {
        cum += b2;
        if (cum + b1 >= (uint32_t)k) {
          d = 1;
        } else {
          cum += b1;
          d = 0;
        }
      }
    }
    prefix |= (uint32_t)(L * 4 + d) << shift;
    above = cum;
    wave_lds_sync();
  }
  return prefix;
}

// Raise the wave's threshold to the k-th largest buffered value and drop the
// entries below it.
__device__ void cand_refresh(Cand& c, int k, int key_bits, uint32_t* hist) {
  const int lane = lane_id();
  int cnts[4] = {c.cnt, 0, 0, 0};
  const float thr = okey_value(wave_kth_key(c.val, 0, cnts, 1, k, key_bits, hist));
  int n = 0;
  for (int base = 0; base < c.cnt; base += 64) {
    const int e = base + lane;
    float v = 0.f;
    int ix = 0;
    bool keep = false;
    if (e < c.cnt) {
      v = c.val[e];
      ix = c.id[e];
      keep = v >= thr;
    }
    wave_lds_sync();
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int pos = n + __popcll(m & lanemask_lt());
      c.val[pos] = v;
      c.id[pos] = ix;
    }
    n += __popcll(m);
    wave_lds_sync();
  }
  c.cnt = n;
  c.thr = thr;
  if (n > kWcap - 64) c.overflow = true;
}

// Offer the 8 values of one step (tokens base..base+7, the first nvalid real).
__device__ void cand_insert(Cand& c, const float v[8], int base, int nvalid, int k, int key_bits, uint32_t* hist) {
  const int lane = lane_id();
  for (int e = 0; e < 8; ++e) {
    if (c.cnt > kWcap - 64) {
      cand_refresh(c, k, key_bits, hist);
      if (c.overflow) return;
    }
    const bool pass = e < nvalid && v[e] >= c.thr;
    const uint64_t m = __ballot(pass);
    if (pass) {
      const int pos = c.cnt + __popcll(m & lanemask_lt());
      c.val[pos] = v[e];
      c.id[pos] = base + e;
    }
    c.cnt += __popcll(m);
  }
  (void)lane;
}

// ------------------------------------------------------------------------------------------
// radix select over a row in global memory (filters the candidate path does not serve)
// ------------------------------------------------------------------------------------------

struct SelectOut {
  uint32_t key;   // selected key
  double w;       // weight of keys >= selected key
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
        const double b3 = __shfl(h3, L), b2 = __shfl(h2, L), b1 = __shfl(h1, L), b0 = __shfl(h0, L);
        int d;
        double wsel;
        if (cum + b3 >= target) {
          d = 3; wsel = cum + b3;
        } else {
          cum += b3;
          if (cum + b2 >= target) {
            d = 2; wsel = cum + b2;
          } else {
            cum += b2;
            if (cum + b1 >= target) {
              d = 1; wsel = cum + b1;
            } else {
              cum += b1;
              d = 0; wsel = cum + b0;
            }
          }
        }
        if (lane == 0) {
          s_u[0] = (uint32_t)(L * 4 + d);
          s_u[1] = 0u;
          s_d[0] = cum;
          s_d[1] = wsel;
        }
      }
    }
    __syncthreads();
    if (s_u[1]) {
      out.reached = false;
      out.key = lo;
      out.w = 0.0;
      __syncthreads();
      return out;
    }
    prefix |= s_u[0] << shift;
    above = s_d[0];
    out.w = s_d[1];
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
// kept set from the candidate buffers
// ------------------------------------------------------------------------------------------

struct Kept {
  float cut;      // keep iff value >= cut
  double mass;    // kept mass
  int n;          // entries in the LDS list (values >= k-th largest)
  bool ok;        // false: list capacity exceeded, use the radix select
};

// Merge the wave buffers of one distribution, find the k-th largest value,
// collect the entries at or above it into the LDS list, weigh them with
// mass(value) in fp64 and apply top-p over whole tie groups.
template <class MassFn>
__device__ Kept kept_from_candidates(float (*cval)[kWcap], int (*cid)[kWcap], const int* wcnt, int k, float top_p,
                                     bool pact, int key_bits, MassFn mass, uint32_t* hist, float* lval, int* lid,
                                     double* lmass, double* red_d, float* red_f, int* s_i) {
  const int tid = threadIdx.x, lane = lane_id();
  Kept out;
  if (tid < 64) {
    const int cnts[4] = {wcnt[0], wcnt[1], wcnt[2], wcnt[3]};
    const float kth = okey_value(wave_kth_key(&cval[0][0], kWcap, cnts, kWaves, k, key_bits, hist));
    int n = 0;
    bool ok = true;
    for (int s = 0; s < kWaves && ok; ++s) {
      for (int base = 0; base < cnts[s]; base += 64) {
        const int e = base + lane;
        const bool keep = e < cnts[s] && cval[s][e] >= kth;
        const uint64_t m = __ballot(keep);
        if (n + __popcll(m) > kListMax) {
          ok = false;
          break;
        }
        if (keep) {
          const int pos = n + __popcll(m & lanemask_lt());
          lval[pos] = cval[s][e];
          lid[pos] = cid[s][e];
        }
        n += __popcll(m);
      }
    }
    if (lane == 0) {
      s_i[0] = ok ? n : -1;
      red_f[0] = kth;
    }
  }
  __syncthreads();
  const int n = s_i[0];
  const float kth = red_f[0];
  __syncthreads();
  if (n < 0) {
    out.ok = false;
    return out;
  }
  out.ok = true;
  out.n = n;
  for (int t = tid; t < n; t += kBlock) lmass[t] = mass(lval[t]);
  __syncthreads();
  double zk = 0.0;
  for (int t = tid; t < n; t += kBlock) zk += lmass[t];
  zk = block_sum_d(zk, red_d);
  float cut = kth;
  if (pact) {
    const double target = (double)top_p * zk;
    float best = -INFINITY;
    for (int t = tid; t < n; t += kBlock) {
      const float v = lval[t];
      double cum = 0.0;
      for (int u = 0; u < n; ++u) cum += (lval[u] >= v) ? lmass[u] : 0.0;
      if (cum >= target) best = __builtin_fmaxf(best, v);
    }
    best = block_max_f(best, red_f);
    cut = (best == -INFINITY) ? kth : best;  // never reached by rounding: keep the whole top-k set
  }
  double zc = 0.0;
  for (int t = tid; t < n; t += kBlock) zc += (lval[t] >= cut) ? lmass[t] : 0.0;
  out.mass = block_sum_d(zc, red_d);
  out.cut = cut;
  return out;
}

// ------------------------------------------------------------------------------------------
// row kernel
// ------------------------------------------------------------------------------------------

struct RowShared {
  float cval[2][kWaves][kWcap];
  int cid[2][kWaves][kWcap];
  uint32_t hist[kWaves][256];
  float lval[kListMax];
  int lid[kListMax];
  double lmass[kListMax];
  double red_d[kWaves];
  float red_f[kWaves];
  uint32_t red_u[kWaves];
  int red_i[kWaves];
  int wcnt[2][kWaves];
  int wovf[2][kWaves];
  double sel_d[2];
  uint32_t sel_u[2];
  int misc[4];
};

template <class LT, bool VEC>
__global__ __launch_bounds__(kBlock) void row_kernel(Args a) {
  __shared__ RowShared sh;
  typedef typename LT::T ET;
  const int N = a.N, G = a.G, V = a.V;
  const int j = blockIdx.x / N, i = blockIdx.x - j * N;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const Req rq = load_req(a, i);
  if (rq.fault || j > rq.gamma) return;
  const size_t row = (size_t)i * (G + 1) + j;
  const ET* lrow = reinterpret_cast<const ET*>(a.logits) + row * (size_t)V;
  RowStats* st = a.stats + row;
  const bool draft_pos = j < rq.gamma;
  const int y = draft_pos ? a.ids[(size_t)i * G + j] : -1;
  const int nsteps = (V + kStep - 1) / kStep;

  if (rq.greedy) {
    // argmax, lowest id among equal maxima; NaN / +inf / no finite value is a fault
    float best = -INFINITY;
    int bidx = -1;
    bool nan = false;
    for (int s = 0; s < nsteps; ++s) {
      const int base = s * kStep + tid * kCh;
      float v[8];
      load_logits<LT, VEC>(lrow, base, V, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) nan |= (v[e] != v[e]);
      const float cm = max8(v);
      if (cm > best) {
        int f = 7;
#pragma unroll
        for (int e = 7; e >= 0; --e)
          if (v[e] == cm) f = e;
        best = cm;
        bidx = base + f;
      }
    }
    const float gbest = block_max_f(best, sh.red_f);
    int cand = (best == gbest && bidx >= 0) ? bidx : INT_MAX;
    cand = block_min_i(cand, sh.red_i);
    const int anynan = block_max_i(nan ? 1 : 0, sh.red_i);
    if (tid == 0) {
      int fault = 0;
      if (anynan || gbest == INFINITY || cand == INT_MAX) fault = kFaultTargetRow;
      RowStats s;
      s.m = gbest;
      s.cut_p = -INFINITY;
      s.cut_q = -INFINITY;
      s.argmax = cand == INT_MAX ? -1 : cand;
      s.z = 0.0;
      s.r = 0.0;
      s.p_y = NAN;
      s.q_y = NAN;
      s.flags = ((draft_pos && y == cand) ? 1 : 0) | (fault << 8);
      s.nlist = -1;
      s.pad[0] = s.pad[1] = 0;
      *st = s;
    }
    return;
  }

  const bool has_q = a.q != nullptr && draft_pos;
  const float* qrow = has_q ? a.q + ((size_t)i * G + j) * (size_t)V : nullptr;
  const float T = rq.T;
  const float c = kLog2e / T;
  const float invT = 1.f / T;
  const bool temper = T != 1.f;
  const bool filt = rq.kact || rq.pact;
  const bool fast = rq.kact && rq.k <= kKFast;

  // ---- one streaming pass over the row pair ----
  float m_t = -FLT_MAX;
  double z_t = 0.0, r_t = 0.0;
  uint32_t qbad = 0u;
  Cand cp{&sh.cval[0][wave][0], &sh.cid[0][wave][0], 0, -INFINITY, false};
  Cand cq{&sh.cval[1][wave][0], &sh.cid[1][wave][0], 0, -INFINITY, false};
  for (int s = 0; s < nsteps; ++s) {
    const int base = s * kStep + tid * kCh;
    float lv[8], qv[8];
    load_logits<LT, VEC>(lrow, base, V, lv);
    if (has_q) load_q<VEC>(qrow, base, V, qv);
    const float cm = max8(lv);
    if (cm > m_t) {
      z_t *= (double)fast_exp2((m_t - cm) * c);
      m_t = cm;
    }
    float zs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) zs += fast_exp2((lv[e] - m_t) * c);
    z_t += (double)zs;
    if (has_q) {
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qbad = max(qbad, __float_as_uint(qv[e]));
        rs += temper ? fast_exp2(fast_log2(qv[e]) * invT) : qv[e];
      }
      r_t += (double)rs;
    }
    if (fast) {
      const int nvalid = VEC ? (base < V ? 8 : 0) : max(0, min(8, V - base));
      if (!cp.overflow && __ballot(cm >= cp.thr)) cand_insert(cp, lv, base, nvalid, rq.k, LT::kKeyBits, sh.hist[wave]);
      if (has_q && !cq.overflow && __ballot(max8(qv) >= cq.thr))
        cand_insert(cq, qv, base, nvalid, rq.k, 32, sh.hist[wave]);
    }
  }

  // ---- block totals ----
  const float m = block_max_f(m_t, sh.red_f);
  const double zpart = z_t * exp2(((double)m_t - (double)m) * (double)c);
  const double Z = block_sum_d(zpart, sh.red_d);
  const double R = has_q ? block_sum_d(r_t, sh.red_d) : 0.0;
  const uint32_t qb = has_q ? block_max_u(qbad, sh.red_u) : 0u;
  int fault = 0;
  if (!(Z > 0.0) || isinf(Z)) fault |= kFaultTargetRow;
  if (has_q && qb >= 0x7f800000u) fault |= kFaultDraftRow;

  float cut_p = -INFINITY, cut_q = -INFINITY;
  double Zk = Z, Rk = R;
  int nlist = -1;
  if (!fault && filt) {
    if (fast && lane == 0) {
      sh.wcnt[0][wave] = cp.cnt;
      sh.wovf[0][wave] = cp.overflow;
      sh.wcnt[1][wave] = cq.cnt;
      sh.wovf[1][wave] = cq.overflow;
    }
    __syncthreads();
    // target
    bool done = false;
    if (fast && !(sh.wovf[0][0] | sh.wovf[0][1] | sh.wovf[0][2] | sh.wovf[0][3])) {
      const double mm = (double)m, TT = (double)T;
      Kept kp = kept_from_candidates(sh.cval[0], sh.cid[0], sh.wcnt[0], rq.k, rq.p, rq.pact, LT::kKeyBits,
                                     [&](float v) { return exp(((double)v - mm) / TT); }, sh.hist[0], sh.lval,
                                     sh.lid, sh.lmass, sh.red_d, sh.red_f, sh.misc);
      if (kp.ok) {
        done = true;
        cut_p = kp.cut;
        Zk = kp.mass;
        nlist = kp.n;
        ListEntry* L = a.lists + row * kLcap;
        for (int t = tid; t < kp.n; t += kBlock) {
          ListEntry e;
          e.id = sh.lid[t];
          e.val = sh.lval[t];
          e.e = sh.lmass[t];
          L[t] = e;
        }
      }
      __syncthreads();
    }
    if (!done) {
      auto kw = [&](int x, uint32_t& key, double& w) {
        const float l = LT::at(lrow, (size_t)x);
        key = okey(l);
        w = (double)fast_exp2((l - m) * c);
      };
      auto kc = [&](int x, uint32_t& key, double& w) {
        key = okey(LT::at(lrow, (size_t)x));
        w = 1.0;
      };
      uint32_t lo = 0u;
      if (rq.kact) lo = block_select(kc, V, 0u, (double)rq.k, LT::kKeyBits, sh.lmass, sh.sel_d, sh.sel_u).key;
      const double zk = rq.kact ? block_sum_above(kw, V, lo, sh.red_d) : Z;
      uint32_t cutk = lo;
      double zc = zk;
      if (rq.pact) {
        SelectOut so = block_select(kw, V, lo, (double)rq.p * zk, LT::kKeyBits, sh.lmass, sh.sel_d, sh.sel_u);
        if (so.reached) {
          cutk = so.key;
          zc = block_sum_above(kw, V, cutk, sh.red_d);
        }
      }
      cut_p = (cutk == 0u) ? -INFINITY : okey_value(cutk);
      Zk = zc;
    }
    // draft
    if (has_q) {
      bool qdone = false;
      if (fast && !(sh.wovf[1][0] | sh.wovf[1][1] | sh.wovf[1][2] | sh.wovf[1][3])) {
        Kept kq = kept_from_candidates(sh.cval[1], sh.cid[1], sh.wcnt[1], rq.k, rq.p, rq.pact, 32,
                                       [&](float v) { return temper_q(v, T); }, sh.hist[0], sh.lval, sh.lid,
                                       sh.lmass, sh.red_d, sh.red_f, sh.misc);
        if (kq.ok) {
          qdone = true;
          cut_q = kq.cut;
          Rk = kq.mass;
        }
        __syncthreads();
      }
      if (!qdone) {
        auto kw = [&](int x, uint32_t& key, double& w) {
          const float q = qrow[x];
          key = okey(q);
          w = temper ? (double)fast_exp2(fast_log2(q) * invT) : (double)q;
        };
        auto kc = [&](int x, uint32_t& key, double& w) {
          key = okey(qrow[x]);
          w = 1.0;
        };
        uint32_t lo = 0u;
        if (rq.kact) lo = block_select(kc, V, 0u, (double)rq.k, 32, sh.lmass, sh.sel_d, sh.sel_u).key;
        const double rk = rq.kact ? block_sum_above(kw, V, lo, sh.red_d) : R;
        uint32_t cutk = lo;
        double rc = rk;
        if (rq.pact) {
          SelectOut so = block_select(kw, V, lo, (double)rq.p * rk, 32, sh.lmass, sh.sel_d, sh.sel_u);
          if (so.reached) {
            cutk = so.key;
            rc = block_sum_above(kw, V, cutk, sh.red_d);
          }
        }
        cut_q = (cutk == 0u) ? -INFINITY : okey_value(cutk);
        Rk = rc;
      }
    }
  }
  if (!fault && has_q && !(Rk > 0.0)) fault |= kFaultDraftMass;

  if (tid == 0) {
    RowStats s;
    s.m = m;
    s.cut_p = cut_p;
    s.cut_q = cut_q;
    s.argmax = -1;
    s.z = Zk;
    s.r = Rk;
    s.p_y = NAN;
    s.q_y = NAN;
    int acc = 0;
    if (draft_pos && !fault) {
      const float ly = LT::at(lrow, (size_t)y);
      const double e = (ly >= cut_p) ? exp(((double)ly - (double)m) / (double)T) : 0.0;
      const double py = e / Zk;
      double qy = 1.0;
      if (a.q != nullptr) {
        const float qv = qrow[y];
        qy = (qv >= cut_q) ? temper_q(qv, T) / Rk : 0.0;
      }
      const double u = (double)a.u_accept[(size_t)i * G + j];
      acc = (u * qy < py) ? 1 : 0;
      s.p_y = py;
      s.q_y = qy;
    }
    s.flags = acc | (fault << 8);
    s.nlist = nlist;
    s.pad[0] = s.pad[1] = 0;
    *st = s;
  }
}

// ------------------------------------------------------------------------------------------
// finish kernel: first rejection, draw, outputs
// ------------------------------------------------------------------------------------------

struct FinShared {
  double wsum[kWaves][kMaxChunks];
  double lw[kLcap];
  int lwid[kLcap];
  double red_d[kWaves];
  int red_i[kWaves];
  int misc[8];
  double miscd[4];
};

// Draw weights of one step (mode 0: p'; 1: max(0, p' - q'); 2: p' with y removed).
template <bool VEC>
__device__ inline void step_weights(const float lv[8], const float qv[8], int base, int mode, float m, float c,
                                    float invZ, float cut_p, float cut_q, float invR, float invT, bool temper, int yA,
                                    float w[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = (lv[e] >= cut_p) ? fast_exp2((lv[e] - m) * c) * invZ : 0.f;
    float x = p;
    if (mode == 1) {
      const float r = temper ? fast_exp2(fast_log2(qv[e]) * invT) : qv[e];
      const float q = (qv[e] >= cut_q) ? r * invR : 0.f;
      x = __builtin_fmaxf(p - q, 0.f);
    } else if (mode == 2) {
      x = (base + e == yA) ? 0.f : p;
    }
    w[e] = x;
  }
}

template <class LT, bool VEC>
__global__ __launch_bounds__(kBlock) void finish_kernel(Args a) {
  __shared__ FinShared sh;
  typedef typename LT::T ET;
  const int G = a.G, V = a.V;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const Req rq = load_req(a, i);
  int32_t* out = a.out_tokens + (size_t)i * (G + 1);
  const RowStats* st = a.stats + (size_t)i * (G + 1);

  int fault = rq.fault, A = 0;
  if (!fault) {
    if (wave == 0) {
      int f = 0;
      for (int jj = lane; jj <= rq.gamma; jj += 64) f |= st[jj].flags >> 8;
      f = wave_or_i(f);
      const bool acc = lane < rq.gamma && (st[lane].flags & 1);
      const uint64_t accm = __ballot(acc);
      const uint64_t within = rq.gamma >= 64 ? ~0ull : ((1ull << rq.gamma) - 1ull);
      const uint64_t rej = ~accm & within;
      if (lane == 0) {
        sh.misc[0] = f;
        sh.misc[1] = rej ? (__ffsll((unsigned long long)rej) - 1) : rq.gamma;
      }
    }
    __syncthreads();
    fault = sh.misc[0];
    A = sh.misc[1];
    __syncthreads();
  }

  if (fault) {
    for (int t = tid; t <= G; t += kBlock) out[t] = -1;
    if (tid == 0) {
      a.out_num[i] = -1;
      if (a.d_fault) a.d_fault[i] = fault;
      if (a.d_resid) a.d_resid[i] = NAN;
    }
    if (a.d_py)
      for (int t = tid; t < G; t += kBlock) a.d_py[(size_t)i * G + t] = NAN;
    if (a.d_qy)
      for (int t = tid; t < G; t += kBlock) a.d_qy[(size_t)i * G + t] = NAN;
    return;
  }

  int z;
  double S_out = NAN;
  if (rq.greedy) {
    z = st[A].argmax;
  } else {
    const RowStats sa = st[A];
    const bool resid = A < rq.gamma;
    const int yA = resid ? a.ids[(size_t)i * G + A] : -1;
    int mode = resid ? (a.q ? 1 : 2) : 0;
    const size_t row = (size_t)i * (G + 1) + A;
    const ET* lrow = reinterpret_cast<const ET*>(a.logits) + row * (size_t)V;
    const float* qrow = (mode == 1) ? a.q + ((size_t)i * G + A) * (size_t)V : nullptr;
    const float T = rq.T;
    const double us = (double)a.u_sample[i];

    if (sa.nlist >= 0) {
      // ---- kept list of row A: all tokens with p' > 0 are in it ----
      const ListEntry* L = a.lists + row * kLcap;
      const int n = sa.nlist;
      double part = 0.0;
      for (int t = tid; t < n; t += kBlock) {
        const ListEntry e = L[t];
        const double p = (e.val >= sa.cut_p) ? e.e / sa.z : 0.0;
        double w = p;
        if (mode == 1) {
          const float qx = qrow[e.id];
          const double q = (qx >= sa.cut_q) ? temper_q(qx, T) / sa.r : 0.0;
          w = p - q > 0.0 ? p - q : 0.0;
        } else if (mode == 2) {
          w = (e.id == yA) ? 0.0 : p;
        }
        sh.lw[t] = w;
        sh.lwid[t] = e.id;
        part += w;
      }
      double S = block_sum_d(part, sh.red_d);
      if (S == 0.0) {
        part = 0.0;
        for (int t = tid; t < n; t += kBlock) {
          const ListEntry e = L[t];
          const double p = (e.val >= sa.cut_p) ? e.e / sa.z : 0.0;
          sh.lw[t] = p;
          part += p;
        }
        S = block_sum_d(part, sh.red_d);
      }
      const double tau = us * S;
      int best = INT_MAX, last = -1;
      for (int t = tid; t < n; t += kBlock) {
        if (!(sh.lw[t] > 0.0)) continue;
        const int id = sh.lwid[t];
        double cum = 0.0;
        for (int u = 0; u < n; ++u) cum += (sh.lwid[u] <= id) ? sh.lw[u] : 0.0;
        if (cum > tau) best = min(best, id);
        last = max(last, id);
      }
      best = block_min_i(best, sh.red_i);
      last = block_max_i(last, sh.red_i);
      z = (best != INT_MAX) ? best : last;
      S_out = S;
    } else {
      // ---- two passes over row A ----
      const float m = sa.m, c = kLog2e / T, invT = 1.f / T;
      const bool temper = T != 1.f;
      const float invZ = (float)(1.0 / sa.z);
      const float invR = (mode == 1) ? (float)(1.0 / sa.r) : 0.f;
      const int nsteps = (V + kStep - 1) / kStep;
      const int spc = (nsteps + kMaxChunks - 1) / kMaxChunks;  // steps per chunk
      const int nch = (nsteps + spc - 1) / spc;
      double S = 0.0;
      int last = -1;
      for (int attempt = 0; attempt < 2; ++attempt) {
        last = -1;
        for (int ch = 0; ch < nch; ++ch) {
          double csum = 0.0;
          for (int s = ch * spc; s < min(nsteps, (ch + 1) * spc); ++s) {
            const int base = s * kStep + tid * kCh;
            float lv[8], qv[8], w[8];
            load_logits<LT, VEC>(lrow, base, V, lv);
            if (mode == 1) load_q<VEC>(qrow, base, V, qv);
            step_weights<VEC>(lv, qv, base, mode, m, c, invZ, sa.cut_p, sa.cut_q, invR, invT, temper, yA, w);
            double ts = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              ts += (double)w[e];
              if (w[e] > 0.f) last = base + e;
            }
            csum += wave_sum_d(ts);
          }
          if (lane == 0) sh.wsum[wave][ch] = csum;
        }
        __syncthreads();
        // chunk totals in a fixed order, then the sum
        if (tid == 0) {
          double tot = 0.0;
          for (int ch = 0; ch < nch; ++ch) tot += ((sh.wsum[0][ch] + sh.wsum[1][ch]) + (sh.wsum[2][ch] + sh.wsum[3][ch]));
          sh.miscd[0] = tot;
        }
        __syncthreads();
        S = sh.miscd[0];
        __syncthreads();
        if (S > 0.0 || mode == 0) break;
        mode = 0;  // zero residual: draw from p'
      }
      last = block_max_i(last, sh.red_i);
      const double tau = us * S;
      // the chunk holding the crossing (serial over at most kMaxChunks totals)
      if (tid == 0) {
        double pre = 0.0;
        int found = -1;
        for (int ch = 0; ch < nch; ++ch) {
          const double cs = (sh.wsum[0][ch] + sh.wsum[1][ch]) + (sh.wsum[2][ch] + sh.wsum[3][ch]);
          if (pre + cs > tau && cs > 0.0) {
            found = ch;
            break;
          }
          pre += cs;
        }
        sh.misc[2] = found;
        sh.miscd[1] = pre;
      }
      __syncthreads();
      const int found = sh.misc[2];
      double pre = sh.miscd[1];
      __syncthreads();
      if (found < 0) {
        z = last;
      } else {
        // walk the steps of the chunk in token order; the crossing is in the
        // last run (thread, step) whose starting prefix is <= tau
        int bestkey = -1, bestz = -1;
        for (int s = found * spc; s < min(nsteps, (found + 1) * spc); ++s) {
          const int base = s * kStep + tid * kCh;
          float lv[8], qv[8], w[8];
          load_logits<LT, VEC>(lrow, base, V, lv);
          if (mode == 1) load_q<VEC>(qrow, base, V, qv);
          step_weights<VEC>(lv, qv, base, mode, m, c, invZ, sa.cut_p, sa.cut_q, invR, invT, temper, yA, w);
          double ts = 0.0;
#pragma unroll
          for (int e = 0; e < 8; ++e) ts += (double)w[e];
          double total;
          const double ex = pre + block_exscan_d(ts, sh.red_d, &total);
          if (ts > 0.0 && ex <= tau) {
            double acc = ex;
            int zz = -1, lastpos = -1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (w[e] > 0.f) lastpos = base + e;
              acc += (double)w[e];
              if (zz < 0 && w[e] > 0.f && acc > tau) zz = base + e;
            }
            bestkey = (s - found * spc) * kBlock + tid;
            bestz = zz >= 0 ? zz : lastpos;
          }
          pre += total;
        }
        const int win = block_max_i(bestkey, sh.red_i);
        if (tid == 0) sh.misc[3] = -1;
        __syncthreads();
        if (win >= 0 && bestkey == win) sh.misc[3] = bestz;
        __syncthreads();
        z = sh.misc[3];
        if (z < 0) z = last;
      }
      S_out = S;
    }
  }

  for (int t = tid; t <= G; t += kBlock) {
    int v = -1;
    if (t < A) v = a.ids[(size_t)i * G + t];
    else if (t == A) v = z;
    out[t] = v;
  }
  if (tid == 0) {
    a.out_num[i] = A;
    if (a.d_fault) a.d_fault[i] = 0;
    if (a.d_resid) a.d_resid[i] = S_out;
  }
  if (a.d_py)
    for (int t = tid; t < G; t += kBlock) a.d_py[(size_t)i * G + t] = (t < rq.gamma && !rq.greedy) ? st[t].p_y : NAN;
  if (a.d_qy)
    for (int t = tid; t < G; t += kBlock) a.d_qy[(size_t)i * G + t] = (t < rq.gamma && !rq.greedy) ? st[t].q_y : NAN;
}

// ------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t stats_bytes(int N, int G) { return align_up((size_t)N * (G + 1) * sizeof(RowStats), 256); }
size_t list_bytes(int N, int G) { return align_up((size_t)N * (G + 1) * kLcap * sizeof(ListEntry), 256); }

struct DeviceBuffer {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<DeviceBuffer> g_ws;  // one per device, grown on demand, kept until exit

template <class LT, bool VEC>
hipError_t launch(const Args& a, hipStream_t stream) {
  const long rows = (long)a.N * (a.G + 1);
  hipLaunchKernelGGL((row_kernel<LT, VEC>), dim3((unsigned)rows), dim3(kBlock), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((finish_kernel<LT, VEC>), dim3((unsigned)a.N), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

int run(int N, int G, int V, const int32_t* ids, const float* q, const void* logits, int dtype,
        const float* temperature, const int32_t* top_k, const float* top_p, const float* u_accept,
        const float* u_sample, int32_t* out_tokens, int32_t* out_num, double* p_y, double* q_y, double* resid,
        int32_t* fault, void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 0 || G < 0 || G > kMaxGamma || V < 1) return SPEC_VERIFY_ERR_SHAPE;
  if (dtype != SPEC_VERIFY_F32 && dtype != SPEC_VERIFY_BF16) return SPEC_VERIFY_ERR_DTYPE;
  if ((long long)N * (G + 1) > 0x7fffffffLL || (long long)V * (G + 1) > (1LL << 40)) return SPEC_VERIFY_ERR_SHAPE;
  if (N == 0) return SPEC_VERIFY_OK;
  if (!logits || !u_sample || !out_tokens || !out_num) return SPEC_VERIFY_ERR_NULL;
  if (G > 0 && (!ids || !u_accept)) return SPEC_VERIFY_ERR_NULL;
  const size_t need = spec_verify_workspace_size(N, G, V);
  if (!workspace) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_VERIFY_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
    DeviceBuffer& b = g_ws[dev];
    if (b.bytes < need) {
      void* p = nullptr;
      // the previous buffer may still be in use by queued work: keep it alive
      if (hipMalloc(&p, need) != hipSuccess) return SPEC_VERIFY_ERR_HIP;
      b.ptr = p;
      b.bytes = need;
    }
    workspace = b.ptr;
    workspace_bytes = b.bytes;
  }
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
  a.stats = reinterpret_cast<RowStats*>(workspace);
  a.lists = reinterpret_cast<ListEntry*>(reinterpret_cast<char*>(workspace) + stats_bytes(N, G));

  // 16-byte vector loads need every row start aligned: V a multiple of 8 and
  // 16-byte aligned base pointers
  const bool vec = (V % 8 == 0) && ((uintptr_t)logits % 16 == 0) && (!q || (uintptr_t)q % 16 == 0);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == SPEC_VERIFY_BF16)
    e = vec ? launch<Bf16, true>(a, s) : launch<Bf16, false>(a, s);
  else
    e = vec ? launch<F32, true>(a, s) : launch<F32, false>(a, s);
  return e == hipSuccess ? SPEC_VERIFY_OK : SPEC_VERIFY_ERR_HIP;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int N, int gmax, int V) {
  (void)V;
  if (N <= 0 || gmax < 0) return 256;
  return stats_bytes(N, gmax) + list_bytes(N, gmax);
}

int spec_verify(int N, int gmax, int V, const int32_t* draft_ids, const float* draft_probs, const void* target_logits,
                int logits_dtype, const float* temperature, const int32_t* top_k, const float* top_p,
                const float* u_accept, const float* u_sample, int32_t* out_tokens, int32_t* out_num_accepted,
                void* workspace, size_t workspace_bytes, void* stream) {
  return run(N, gmax, V, draft_ids, draft_probs, target_logits, logits_dtype, temperature, top_k, top_p, u_accept,
             u_sample, out_tokens, out_num_accepted, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes,
             stream);
}

int spec_verify_diag(int N, int gmax, int V, const int32_t* draft_ids, const float* draft_probs,
                     const void* target_logits, int logits_dtype, const float* temperature, const int32_t* top_k,
                     const float* top_p, const float* u_accept, const float* u_sample, int32_t* out_tokens,
                     int32_t* out_num_accepted, double* p_y, double* q_y, double* resid_mass, int32_t* fault,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return run(N, gmax, V, draft_ids, draft_probs, target_logits, logits_dtype, temperature, top_k, top_p, u_accept,
             u_sample, out_tokens, out_num_accepted, p_y, q_y, resid_mass, fault, workspace, workspace_bytes, stream);
}

const char* spec_verify_status_string(int status) {
  switch (status) {
    case SPEC_VERIFY_OK: return "ok";
    case SPEC_VERIFY_ERR_NULL: return "a required pointer is NULL";
    case SPEC_VERIFY_ERR_SHAPE: return "N, gmax or V out of range";
    case SPEC_VERIFY_ERR_DTYPE: return "unknown logits dtype";
    case SPEC_VERIFY_ERR_WORKSPACE: return "workspace smaller than spec_verify_workspace_size";
    case SPEC_VERIFY_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int spec_verify_version(void) { return 1; }

}  // extern "C"
