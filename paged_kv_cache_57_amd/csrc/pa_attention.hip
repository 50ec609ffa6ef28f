// Paged attention for gfx950: planner, VALU and MFMA workers, log-sum-exp merge.
//
// What is computed: out = softmax(q Kᵀ · scale) V over each sequence's
// visible keys ("第7章：大模型部署实战" §2.2.2 formula; "第 15 章：推理引擎与部署"
// §15.1), with the keys and values gathered page by page through the block
// table ("第 15 章" §15.6 "PagedAttention：分页 KV Cache").
//
// How:
//  * A one-workgroup planner reads query_start_loc / context_lens, checks
//    them, and turns every sequence into work items.  An item is a key
//    partition (a fixed range of key positions) of either
//      - one query row and one query head (VALU class: float32 batches and
//        bfloat16 single-row decodes with one query head per KV head),
//      - a tile of 16 query rows that share one KV head (MFMA class: bfloat16
//        sequences with at most 16 rows, where a row is one query position
//        of one of the G query heads of a KV head, e.g. GQA decodes), or
//      - a tile of 256 such rows (TILE class: bfloat16 prefill chunks).
//    Partition sizes depend only on the sequence's own lengths, so a
//    sequence's result does not depend on the rest of the batch.
//  * Persistent workers walk the items, with a fixed stride (wave w takes
//    items w, w + W, w + 2W, ...) or from ticket counters (the TILE worker, and
//    the VALU worker in batches without shared pages).  Each item streams its
//    pages with 16-byte loads and keeps the running max m, the
//    running sum l and the unnormalised output O of the tiled online softmax
//    ("第 15 章" §15.1 "算法详解": m_new = max(m, rowmax S), α = exp(m − m_new),
//    P = exp(S − m_new), l = αl + rowsum P, O = diag(α)O + PV), in base 2
//    (scale · log2 e folded into the scores, exp2 in hardware).
//  * A context split into several partitions is merged by rescaling the
//    partial states to the common maximum — the same α step applied to
//    finished states: M = max m_p, l = Σ l_p 2^(m_p − M), O = Σ O_p 2^(m_p − M) / l.
//    The pages name split-K decoding for long contexts ("大模型部署.md" §2.5
//    item 2, TurboMind) without giving its math; this merge is the
//    rescaling rule above.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

enum { CLS_NONE = 0, CLS_VALU = 1, CLS_MFMA = 2, CLS_TILE = 3 };
constexpr int kPartValu = 1024;         // keys per VALU partition
constexpr int kPartMfmaDecode = 256;    // keys per partition of a one-row GQA decode tile
constexpr int kPartMfmaPrefill = 1024;  // keys per partition of a small multi-row tile
constexpr int kPartTile = 1024;         // keys per partition of a 256-row tile
constexpr int kTileRows = 16;           // query rows per MFMA item
constexpr int kTileWaves = 8;           // wavefronts per TILE workgroup, 32 rows each
constexpr int kTileStages = 4;          // LDS stages of the TILE worker's load pipeline (2 per barrier)
constexpr int kBigRows = 32 * kTileWaves;  // query rows per TILE item
constexpr int kMaxWorkerGroups = 2048;  // persistent workgroups per worker launch
constexpr int kMaxTileGroups = 256;     // TILE workgroups (one per compute unit)
constexpr int kXcds = 8;                // XCDs (each with its own L2); TILE items are sliced per XCD
constexpr int kHwRegXccId = (3 << 11) | 20;  // s_getreg operand: HW_REG_XCC_ID, bits 3:0
constexpr int kValuGridPerResident = 4;  // VALU grid: this many times the resident workgroups
constexpr int kValuTicket = 64;         // ctrl word of the VALU ticket counter (bytes 256..259 of the workspace)
constexpr float kLazyRescale = 8.f;     // MFMA and TILE workers: raise the exponent reference only past this growth (log2)
constexpr int kMergeSplitParts = 32;    // partitions per row from which four wavefronts merge a row
constexpr float kNegInf = -INFINITY;


// floats per partial state: O[D], m, l, padded to keep 16-byte alignment
__host__ __device__ constexpr int slot_floats(int D) { return D + 4; }

struct SeqWork {
  int cls;
  int part;    // keys per partition
  int nparts;  // partitions of the context
  int groups;  // items per partition index: rows x heads (VALU) or tiles x KV heads (MFMA)
};

__host__ __device__ inline SeqWork seq_work(bool is_f32, int G, int Hq, int Hkv, int q_len, int L) {
  SeqWork w{CLS_NONE, 1, 0, 0};
  if (q_len <= 0 || L <= 0) return w;
  const int rows = q_len * G;  // rows of one KV head: positions x query heads of the group
  if (is_f32 || (G == 1 && q_len == 1)) {
    w.cls = CLS_VALU;
    w.part = kPartValu;
    w.groups = q_len * Hq;
  } else if (rows <= kTileRows) {
    w.cls = CLS_MFMA;
    w.part = q_len == 1 ? kPartMfmaDecode : kPartMfmaPrefill;
    w.groups = Hkv;
  } else {
    w.cls = CLS_TILE;
    w.part = kPartTile;
    w.groups = ((rows + kBigRows - 1) / kBigRows) * Hkv;
  }
  w.nparts = (L + w.part - 1) / w.part;
  return w;
}

// A shared-prefix group entry: its members' rows over the S shared keys, in
// partitions of the one-row decode size (the group's rows are decode rows,
// and short partitions spread its keys over many wavefronts).
__host__ __device__ inline SeqWork group_work(int Hkv, int S) {
  SeqWork w{CLS_MFMA, kPartMfmaDecode, 0, Hkv};
  w.nparts = (S + kPartMfmaDecode - 1) / kPartMfmaDecode;
  return w;
}

// Smallest partition any sequence of this batch can use (bounds the partial states).
inline int min_part(bool is_f32, int G) {
  if (is_f32) return kPartValu;
  const int m = G == 1 ? kPartValu : kPartMfmaDecode;
  return std::min(m, std::min(kPartMfmaPrefill, kPartTile));
}

struct AttnParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* qsl;
  int32_t mbps;
  int32_t num_seqs, T, max_q_len, max_ctx;
  int32_t Hq, Hkv, G, num_blocks;
  float scale_log2;
  int32_t is_f32;
  int32_t* ctrl;  // [2] VALU items, [3] MFMA items, [4] TILE items, [5] rows to merge, [6] some sequence
                  // shares pages with a neighbour, [7] VALU items before the last partitions, [8..15]
                  // TILE tickets per XCD slice, [16] sequences in perm_b, [17] VALU tickets in the
                  // length order, [kValuTicket] VALU tickets (on a 256-byte line of its own)
  int32_t* pre_v;  // exclusive prefix over sequences of VALU items, [S + 1]
  int32_t* pre_m;  // ... of MFMA items
  int32_t* pre_t;  // ... of TILE items
  int32_t* pre_g;  // ... of (query token, query head) rows whose context was split
  // VALU items in ticket order (batches with no shared pages): first every item that is not
  // its row's last partition, numbered through pre_a (exclusive prefix over entries of
  // rows x heads x (partitions - 1)); then the last partitions, sequence by sequence in
  // perm_b order (longest last partition first, in 16 classes of length), numbered through
  // pre_b (exclusive prefix of rows x heads over perm_b).  seq_aux: per sequence, its
  // length class (-1: no VALU items) and its rows x heads, from the planner's first pass.
  int32_t* pre_a;
  int32_t* pre_b;
  int32_t* perm_b;
  int32_t* seq_aux;
  i32x4* seqinfo;  // per entry: first query row, q_len, context length, flags (kEnt*)
  float* partials;  // [T][Hq][maxparts][D + 4]: O (unnormalised), m, l, 2 pad
  int32_t maxparts;
  int32_t* dev_status;
  // Shared prefixes: entries [num_seqs, num_ent) stand for the groups of
  // `groups` ([num_groups][3]: first sequence, members, shared keys).
  int32_t num_ent;
  const int32_t* groups;
  int32_t num_groups;
  i32x4* seqx;  // per entry: key offset, shared partitions before the own ones, member flag, table row
  // One-pass GQA decode: completion counters per (sequence, KV head) and the call's tag.
  unsigned long long* dec_ctr;
  uint32_t call_tag;
  // VALU worker: workgroups resident on the device at once (at most the grid)
  int32_t valu_resident;
  // the host's bound on VALU items allows the length order (fewer than kLenOrderItems per
  // resident wavefront): the planner then records what the order needs
  int32_t len_order_ok;
};

// Entry flags.  A group entry's rows are its members' single decode rows,
// all at the last position of the shared keys (every row sees all of them);
// its partitions fill the members' partial slots 0 .. nps-1.  A member
// skips the shared keys and numbers its own partitions from nps on.
constexpr int kEntValid = 1, kEntGroup = 2, kEntMember = 4;
// kEntShared: the sequence's first page is also the first page of the sequence
// before or after it in the batch (forked branches of one prompt, beams):
// their pages are read by several sequences of the pass, so its workers load
// them with plain loads that let the other reads hit in the caches.
constexpr int kEntShared = 8;

struct SeqInfo {
  int a, q_len, L, flags;
  bool ok;
};

// Checks one sequence's row range and length against the host-known bounds.
__device__ inline SeqInfo read_seq(const AttnParams& p, int s) {
  SeqInfo si;
  si.a = p.qsl[s];
  const int b = p.qsl[s + 1];
  si.q_len = b - si.a;
  si.L = p.context_lens[s];
  si.ok = si.a >= 0 && b >= si.a && b <= p.T && si.q_len <= p.max_q_len && si.L >= 0 &&
          si.L <= p.max_ctx && si.q_len <= si.L && (si.L + kBlock - 1) / kBlock <= p.mbps;
  si.flags = si.ok ? kEntValid : 0;
  return si;
}

// Key offset, shared partitions and table row of an entry (all 0 / s without groups).
struct EntX {
  int koff, nps, trow;
};
__device__ inline EntX ent_x(const AttnParams& p, int s, int flags) {
  EntX x{0, 0, s};
  if (flags & (kEntGroup | kEntMember)) {
    const i32x4 v = p.seqx[s];
    x.koff = __builtin_amdgcn_readfirstlane(v[0]);
    x.nps = __builtin_amdgcn_readfirstlane(v[1]);
    if (flags & kEntGroup) x.trow = __builtin_amdgcn_readfirstlane(v[3]);
  }
  return x;
}

// The planner's record of sequence s, as wave-uniform values (one 16-byte load).
__device__ inline SeqInfo seq_record(const AttnParams& p, int s) {
  const i32x4 v = p.seqinfo[s];
  SeqInfo si;
  si.a = __builtin_amdgcn_readfirstlane(v[0]);
  si.q_len = __builtin_amdgcn_readfirstlane(v[1]);
  si.L = __builtin_amdgcn_readfirstlane(v[2]);
  si.flags = __builtin_amdgcn_readfirstlane(v[3]);
  si.ok = (si.flags & kEntValid) != 0;
  return si;
}

// Item -> sequence lookup.  Every workgroup of a worker first copies every
// stride-th entry of the item prefix array into LDS (at most kSkip entries;
// stride 1 for batches of fewer than kSkip sequences), so that finding the
// sequence of an item costs LDS probes instead of a chain of dependent
// global loads; only batches larger than kSkip sequences finish the search
// in global memory, inside one stride.
constexpr int kSkip = 2048;
constexpr int kLenClasses = 16;  // length classes of the VALU worker's last partitions
constexpr int kLenOrderItems = 8;  // the length order is used below this many VALU items per resident wavefront

struct SkipTable {
  int stride, count;
};

__device__ inline SkipTable stage_skip(int* sk, const int32_t* pre, int n) {
  SkipTable t;
  t.stride = (n + kSkip) / kSkip;  // ceil((n + 1) / kSkip)
  t.count = n / t.stride + 1;      // entries i * stride <= n
#pragma unroll 8
  for (int i0 = 0; i0 < t.count; i0 += (int)blockDim.x) {
    const int i = min(i0 + (int)threadIdx.x, t.count - 1);  // threads past the end repeat the last entry
    sk[i] = pre[i * t.stride];
  }
  __syncthreads();
  return t;
}

struct SeqHit {
  int s, first;  // sequence, and pre[s]: its first item
};

// Largest s in [0, n) with pre[s] <= x, for pre non-decreasing with
// pre[0] <= x < pre[n] and x wave-uniform.
__device__ inline SeqHit find_seq(const int* sk, SkipTable t, const int32_t* pre, int n, int x) {
  int lo = 0, hi = t.count, vlo = 0;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    const int v = __builtin_amdgcn_readfirstlane(sk[mid]);
    if (v <= x) {
      lo = mid;
      vlo = v;
    } else {
      hi = mid;
    }
  }
  vlo = __builtin_amdgcn_readfirstlane(sk[lo]);
  int a = lo * t.stride, b = min(a + t.stride, n);
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    const int v = pre[mid];
    if (v <= x) {
      a = mid;
      vlo = v;
    } else {
      b = mid;
    }
  }
  return SeqHit{a, vlo};
}

// ---------------------------------------------------------------- planner
// One workgroup: checks every sequence, records it, and writes the exclusive
// prefix sums of its items per worker class and of its rows to merge; for small
// batches also the VALU worker's length order (a second pass: a counting sort of
// the sequences by the length of their last partition).
__device__ inline i32x4 wave_incl_scan(i32x4 v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    i32x4 y;
    y[0] = __shfl_up(v[0], o, 64);
    y[1] = __shfl_up(v[1], o, 64);
    y[2] = __shfl_up(v[2], o, 64);
    y[3] = __shfl_up(v[3], o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

__device__ inline int wave_incl_scan1(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}

// With shared-prefix groups it first checks every group — one wavefront per
// group, the lanes comparing the members' table entries with the first
// member's — and records the group entries and the members' offsets; a group
// that fails a check is dropped (its members are attended as plain
// sequences) and PA_DEV_BAD_GROUP is set.
__device__ inline void plan_groups(const AttnParams& p, int tid) {
  for (int s = tid; s < p.num_seqs; s += 1024) p.seqx[s] = i32x4{0, 0, 0, 0};
  __syncthreads();  // members are marked below, after every entry has been cleared
  const int lane = tid & 63;
  for (int g = tid >> 6; g < p.num_groups; g += 16) {
    const int first = p.groups[3 * g], n = p.groups[3 * g + 1], S = p.groups[3 * g + 2];
    // in increasing order without overlap, 2..16/G members inside the batch, whole shared pages
    const bool after_prev = g == 0 || (int64_t)first >= (int64_t)p.groups[3 * g - 3] + p.groups[3 * g - 2];
    const bool shape = after_prev && n >= 2 && n <= kTileRows && n * p.G <= kTileRows && first >= 0 &&
                       first <= p.num_seqs - n && S > 0 && S % kBlock == 0 && S <= p.max_ctx;
    bool bad = !shape;
    if (shape) {
      const SeqInfo si = read_seq(p, first + min(lane, n - 1));
      bad = !si.ok || si.q_len != 1 || si.L < S;
      const int nb = S / kBlock;  // <= mbps, as S <= max_ctx
      const int64_t cmp = (int64_t)(n - 1) * nb;
      const int32_t* lead = p.block_tables + (int64_t)first * p.mbps;
      bool diff = false;  // no short circuit: the loads of all iterations are independent
#pragma unroll 4
      for (int64_t i = lane; i < cmp; i += 64) {
        const int m = 1 + (int)(i / nb), j = (int)(i % nb);
        diff |= p.block_tables[(int64_t)(first + m) * p.mbps + j] != lead[j];
      }
      bad = bad || diff;
    }
    const bool good = __builtin_amdgcn_ballot_w64(bad) == 0;
    const int nps = good ? group_work(p.Hkv, S).nparts : 0;
    if (good && lane < n) p.seqx[first + lane] = i32x4{S, nps, 1, 0};
    if (lane == 0) {
      if (!good) flag_status(p.dev_status, PA_DEV_BAD_GROUP);
      p.seqinfo[p.num_seqs + g] = i32x4{good ? p.qsl[first] : 0, n, S, good ? (kEntValid | kEntGroup) : 0};
      p.seqx[p.num_seqs + g] = i32x4{0, 0, 0, good ? first : 0};
    }
  }
}

__global__ __launch_bounds__(1024) void plan_kernel(AttnParams p) {
  __shared__ i32x4 wsum[16];
  __shared__ int wsum_a[16];
  __shared__ i32x4 carry;
  __shared__ int carry_a;
  __shared__ int any_shared;
  // last partitions: sequences and rows x heads per length class, the classes' first slots
  // (longest class first), and the running (sequences << 32 | rows x heads) per class
  __shared__ int cls_n[kLenClasses], cls_g[kLenClasses], cls_n0[kLenClasses], cls_g0[kLenClasses];
  __shared__ unsigned long long cls_run[kLenClasses];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid < kLenClasses) {
    cls_n[tid] = 0;
    cls_g[tid] = 0;
    cls_run[tid] = 0;
  }
  if (tid == 0) {
    carry = i32x4{0, 0, 0, 0};
    carry_a = 0;
    any_shared = 0;
    if (p.qsl[0] != 0 || p.qsl[p.num_seqs] != p.T) flag_status(p.dev_status, PA_DEV_BAD_LENGTH);
  }
  if (p.num_groups > 0) plan_groups(p, tid);
  __syncthreads();
  for (int base = 0; base < p.num_ent; base += 1024) {
    const int s = base + tid;
    i32x4 cnt = {0, 0, 0, 0};  // VALU, MFMA, TILE items, rows to merge
    int cnt_a = 0;  // VALU items that are not their row's last partition
    if (s < p.num_seqs) {
      if (p.len_order_ok) p.seq_aux[2 * s] = -1;
      SeqInfo si = read_seq(p, s);
      int koff = 0, nps = 0;
      if (p.num_groups > 0) {
        const i32x4 x = p.seqx[s];
        if (x[2]) {
          koff = x[0];
          nps = x[1];
          si.flags |= kEntMember;
        }
      }
      if (si.ok && si.L > 0) {
        const int32_t first = p.block_tables[(int64_t)s * p.mbps];
        const bool prev = s > 0 && p.context_lens[s - 1] > 0 && p.block_tables[(int64_t)(s - 1) * p.mbps] == first;
        const bool next = s + 1 < p.num_seqs && p.context_lens[s + 1] > 0 &&
                          p.block_tables[(int64_t)(s + 1) * p.mbps] == first;
        if (prev || next) {
          si.flags |= kEntShared;
          any_shared = 1;  // every writer stores the same value
        }
      }
      p.seqinfo[s] = i32x4{si.a, si.q_len, si.L, si.flags};
      if (!si.ok) {
        flag_status(p.dev_status, PA_DEV_BAD_LENGTH);
      } else {
        const SeqWork w = seq_work(p.is_f32, p.G, p.Hq, p.Hkv, si.q_len, si.L - koff);
        const int items = w.groups * w.nparts;
        if (w.cls == CLS_VALU) {
          cnt[0] = items;
        }
        if (w.cls == CLS_VALU && p.len_order_ok) {
          cnt_a = items - w.groups;
          // length class of the last partition (of the last row): longer ones are handed out first
          const int tail = (si.L - koff - 1) % w.part + 1;
          const int c = (tail - 1) * kLenClasses / w.part;
          p.seq_aux[2 * s] = c;
          p.seq_aux[2 * s + 1] = w.groups;
          atomicAdd(&cls_n[c], 1);
          atomicAdd(&cls_g[c], w.groups);
        }
        else if (w.cls == CLS_MFMA) cnt[1] = items;
        else if (w.cls == CLS_TILE) cnt[2] = items;
        if (nps > 0 || w.nparts > 1) cnt[3] = si.q_len * p.Hq;
      }
    } else if (s < p.num_ent) {
      const i32x4 r = p.seqinfo[s];  // a group entry, recorded by plan_groups
      if (r[3] & kEntGroup) {
        const SeqWork w = group_work(p.Hkv, r[2]);
        cnt[1] = w.groups * w.nparts;
      }
    }
    const i32x4 inc = wave_incl_scan(cnt, lane);
    const int inc_a = wave_incl_scan1(cnt_a, lane);
    if (lane == 63) {
      wsum[wv] = inc;
      wsum_a[wv] = inc_a;
    }
    __syncthreads();
    i32x4 before = carry;
    int before_a = carry_a;
    for (int k = 0; k < wv; ++k) {
      before += wsum[k];
      before_a += wsum_a[k];
    }
    if (s < p.num_ent) {
      const i32x4 ex = before + inc - cnt;
      p.pre_v[s] = ex[0];
      p.pre_m[s] = ex[1];
      p.pre_t[s] = ex[2];
      p.pre_g[s] = ex[3];
      p.pre_a[s] = before_a + inc_a - cnt_a;
    }
    __syncthreads();
    if (tid == 0) {
      i32x4 tot = carry;
      int tot_a = carry_a;
      for (int k = 0; k < 16; ++k) {
        tot += wsum[k];
        tot_a += wsum_a[k];
      }
      carry = tot;
      carry_a = tot_a;
    }
    __syncthreads();
  }
  // The length order pays where the VALU items are few per resident wavefront (a small
  // batch's last round of items is most of its time); in a large batch the items left at the
  // end are a small share and the planner's second pass would cost more than it saves.
  const bool by_len = p.len_order_ok && any_shared == 0 && carry[0] < kLenOrderItems * p.valu_resident;
  if (tid == 0) p.ctrl[17] = by_len ? 1 : 0;
  if (by_len) {
    // the classes' first slots, longest class first
    if (tid == 0) {
      int n0 = 0, g0 = 0;
      for (int c = kLenClasses - 1; c >= 0; --c) {
        cls_n0[c] = n0;
        cls_g0[c] = g0;
        n0 += cls_n[c];
        g0 += cls_g[c];
      }
      p.pre_b[n0] = g0;
      p.ctrl[16] = n0;
    }
    __syncthreads();
    // each sequence with VALU items takes the next slot of its class (one atomic gives its
    // slot and the rows x heads before it in the class together, so pre_b stays increasing)
    for (int s = tid; s < p.num_seqs; s += 1024) {
      const int c = p.seq_aux[2 * s];  // written by this thread in the first pass
      if (c >= 0) {
        const unsigned long long g = (unsigned long long)p.seq_aux[2 * s + 1];
        const unsigned long long r = atomicAdd(&cls_run[c], (1ull << 32) | g);
        const int k = cls_n0[c] + (int)(r >> 32);
        p.perm_b[k] = s;
        p.pre_b[k] = cls_g0[c] + (int)(r & 0xffffffffu);
      }
    }
  }
  if (tid == 0) {
    p.pre_v[p.num_ent] = carry[0];
    p.pre_m[p.num_ent] = carry[1];
    p.pre_t[p.num_ent] = carry[2];
    p.pre_g[p.num_ent] = carry[3];
    p.ctrl[2] = carry[0];
    p.ctrl[3] = carry[1];
    p.ctrl[4] = carry[2];
    p.ctrl[5] = carry[3];
    p.ctrl[6] = any_shared;
    p.pre_a[p.num_ent] = carry_a;
    p.ctrl[7] = carry_a;
    for (int x = 0; x < kXcds; ++x) p.ctrl[8 + x] = 0;  // TILE tickets handed out so far, per XCD slice
    p.ctrl[kValuTicket] = 0;                             // VALU tickets handed out so far
  }
}

// Work distribution and control flow in the workers: a wavefront walks the
// items wave_id, wave_id + nwaves, ... (or takes them from a ticket counter,
// below) with the item made uniform by readfirstlane, and nothing inside an
// item branches on the lane index.  Lane-dependent branches around the loop
// (for example "lane 0 fetches the next item, then everyone reads it back")
// were merged by the compiler across the loop's back edge into an inner loop
// that only lane 0 leaves, after which the other lanes ran on with a stale
// item and read lane values of a lane that was no longer active.  So stores
// are unconditional (lanes holding the same value write the same address),
// loads use clamped, always-valid indices, and a ticket is taken by thread 0
// between two workgroup barriers and read back from LDS.
__device__ inline int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Physical block ids of this partition's pages: lane j holds page j (lanes
// past the last page repeat it).  An id outside the pool is replaced by block
// 0, which keeps every address inside the pool, and PA_DEV_BAD_BLOCK is set.
__device__ inline int load_block_ids(const AttnParams& p, int s, int first_blk, int nblk, int lane) {
  const int j = min(lane, nblk - 1);
  const int bid = p.block_tables[(int64_t)s * p.mbps + first_blk + j];
  const bool bad = bid < 0 || bid >= p.num_blocks;
  if (__builtin_amdgcn_ballot_w64(bad)) flag_status(p.dev_status, PA_DEV_BAD_BLOCK);
  return bad ? 0 : bid;
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- VALU worker
// One wavefront per item: one query row x one query head x one key partition.
// Workgroups of one wavefront, as many as fit on the GPU at once, walk the items
// (see the item loop for their order).
// Keys are processed 64 at a time (4 pages).  Lane layout of a key page
// [D/X][16][X]: load i of page j gives lane l the 16-byte group 4i + l/16 of
// key l%16, so each lane accumulates a partial dot over D/4 elements and two
// exchanges (lanes ±32, ±16) finish the four pages' dots, leaving lane l with
// the score of key l of the 64.  Value pages [D][16] give lane l, in load i,
// X consecutive keys of one value column, so P·V accumulates in-lane and only
// the lanes sharing a column are summed at the end.
template <typename T, int D>
__global__ __launch_bounds__(64) void valu_attn_kernel(AttnParams p) {
  constexpr int X = Elem<T>::X;
  constexpr int NCH = D / X;   // 16-byte groups per key row
  constexpr int NIK = NCH / 4; // key loads per page
  constexpr int LPR = 16 / X;  // lanes per value column
  constexpr int RPI = 64 / LPR;  // value columns per load
  constexpr int NIV = D / RPI;   // value loads per page
  constexpr bool kBf16 = sizeof(T) == 2;
  __shared__ float lds_p[64];
  __shared__ int skip[kSkip], skip_b[kSkip];
  __shared__ int ticket;
  __shared__ int order_b[5];  // ticket order: items before the last partitions, sequences in
                              // perm_b, skip_b's stride and count, perm_b - pre_b (kept here,
                              // not in scalar registers)

  const int lane = threadIdx.x & 63;
  const int total = wave_uniform(p.ctrl[2]);
  // Items.  In a batch where sequences share pages with a neighbour (branches of one
  // prompt), workgroup b takes items π(b), π(b) + grid, ... in the planner's sequence
  // order (pre_v: a sequence's items row-head by row-head, partitions innermost), and the
  // grid is a few times the resident workgroups, so items start in dispatch order.  π
  // permutes each block of 32 workgroups so that XCD x (workgroups go to the XCDs in turn)
  // takes items 4x .. 4x + 3 of the block.  The readers of a page (one head and partition
  // in neighbouring sequences, Hq x partitions items apart: a multiple of 32 for 32 query
  // heads) then run close in time on one XCD and share its reads through L2.  Otherwise
  // only the resident workgroups work: b takes item b, then the resident count plus a
  // ticket from one counter, so every wavefront stays busy to the end whatever the mix of
  // item lengths.  Tickets follow the sequence order too, except in batches with few items
  // per resident wavefront, where the planner orders the rows' last partitions after all
  // other items, longest first (pre_a, pre_b), so that the items left at the end are the
  // short ones.  Thread 0 takes the ticket between two barriers (the workgroup is this one
  // wavefront), so no lane-dependent branch spans the item loop.
  const bool strided = wave_uniform(p.ctrl[6]) != 0;
  const int b = (int)blockIdx.x;
  // no first item (its block of 32 starts past the end) or, with tickets, not resident: no work
  if ((b & ~31) >= total || (!strided && b >= p.valu_resident)) return;
  const bool by_len = !strided && wave_uniform(p.ctrl[17]) != 0;  // the planner's length order
  const int32_t* const pre = by_len ? p.pre_a : p.pre_v;  // the items' prefix over sequences
  const SkipTable tab = stage_skip(skip, pre, p.num_ent);
  if (by_len) {
    const int num_b = wave_uniform(p.ctrl[16]);
    const SkipTable tb = stage_skip(skip_b, p.pre_b, num_b);
    order_b[0] = p.ctrl[7];  // every lane stores the same values
    order_b[1] = num_b;
    order_b[2] = tb.stride;
    order_b[3] = tb.count;
    order_b[4] = (int)(p.perm_b - p.pre_b);
  }
  const T* __restrict__ kc = (const T*)p.k_cache;
  const T* __restrict__ vc = (const T*)p.v_cache;
  const int64_t page_elems = (int64_t)kBlock * D;

  for (int item = wave_uniform(strided ? (b & ~31) + 4 * (b & 7) + ((b >> 3) & 3) : b); item < total;) {
    // the item's sequence, row-head (rh) and partition
    int s, local;
    const int total_a = by_len ? wave_uniform(order_b[0]) : total;
    const bool last_part = item >= total_a;  // wave-uniform; never in sequence order
    if (!last_part) {
      const SeqHit hit = find_seq(skip, tab, pre, p.num_ent, item);
      s = hit.s;
      local = item - hit.first;
    } else {
      const SkipTable tb{wave_uniform(order_b[2]), wave_uniform(order_b[3])};
      const SeqHit hit = find_seq(skip_b, tb, p.pre_b, wave_uniform(order_b[1]), item - total_a);
      s = wave_uniform(p.pre_b[wave_uniform(order_b[4]) + hit.s]);  // perm_b[hit.s]
      local = item - total_a - hit.first;
    }
    const SeqInfo si = seq_record(p, s);
    const EntX ex = ent_x(p, s, si.flags);  // a member skips the shared keys
    const SeqWork w = seq_work(p.is_f32, p.G, p.Hq, p.Hkv, si.q_len, si.L - ex.koff);
    // sequence order: partitions innermost; ticket order: the partitions before the last,
    // innermost, or the last partition of row-head `local`
    // (in the length order an item before the last partitions has 2 or more in its sequence)
    const int np = by_len ? max(w.nparts - 1, 1) : w.nparts;
    const int pidx = last_part ? w.nparts - 1 : local % np;
    const int rh = last_part ? local : local / np;
    const int h = rh % p.Hq;
    const int i = rh / p.Hq;
    const int t = si.a + i;
    const int pos = si.L - si.q_len + i;
    const int g = h / p.G;
    const int kv_lo = ex.koff + pidx * w.part;
    const int kv_hi = min(kv_lo + w.part, pos + 1);

    float m = kNegInf, lsum = 0.f;
    float acc[NIV];
#pragma unroll
    for (int k = 0; k < NIV; ++k) acc[k] = 0.f;

    auto attend = [&](auto stream_tag) {
      constexpr bool kStream = decltype(stream_tag)::value;
      const int nblk = (kv_hi - kv_lo + kBlock - 1) / kBlock;
      const int bidv = load_block_ids(p, s, kv_lo / kBlock, nblk, lane);

      // q row: the 16-byte groups this lane multiplies
      const T* qrow = (const T*)p.q + ((int64_t)t * p.Hq + h) * D;
      u32x4 qv[NIK];
#pragma unroll
      for (int k = 0; k < NIK; ++k) qv[k] = ld16(qrow + (4 * k + (lane >> 4)) * X);

      for (int base = kv_lo; base < kv_hi; base += 64) {
        const int j0 = (base - kv_lo) >> 4;
        u32x4 kr[4][NIK], vr[4][NIV];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (base + kBlock * j < kv_hi) {
            const int bid = readlane(bidv, j0 + j);
            const int64_t page = ((int64_t)bid * p.Hkv + g) * page_elems;
            const T* kp = kc + page;
            const T* vp = vc + page;
#pragma unroll
            for (int k = 0; k < NIK; ++k)
              kr[j][k] = ld16_page<kStream>(kp + ((4 * k + (lane >> 4)) * kBlock + (lane & 15)) * X);
#pragma unroll
            for (int k = 0; k < NIV; ++k)
              vr[j][k] = ld16_page<kStream>(vp + (RPI * k + lane / LPR) * kBlock + (lane % LPR) * X);
          } else {
#pragma unroll
            for (int k = 0; k < NIK; ++k) kr[j][k] = u32x4{0, 0, 0, 0};
#pragma unroll
            for (int k = 0; k < NIV; ++k) vr[j][k] = u32x4{0, 0, 0, 0};
          }
        }
        // partial dots of this lane's key (lane % 16) in each of the 4 pages
        float kd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float d = 0.f;
#pragma unroll
          for (int k = 0; k < NIK; ++k) {
            if constexpr (kBf16) {
#pragma unroll
              for (int e = 0; e < 4; ++e) d = dot2_bf16(kr[j][k][e], qv[k][e], d);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                d = fmaf(__uint_as_float(kr[j][k][e]), __uint_as_float(qv[k][e]), d);
            }
          }
          kd[j] = d;
        }
        // finish the dots across the four lane groups: lane l ends with key l
        const bool up2 = lane & 32, up1 = lane & 16;
        float keep0 = up2 ? kd[2] : kd[0], keep1 = up2 ? kd[3] : kd[1];
        keep0 += shfl_xor_f(up2 ? kd[0] : kd[2], 32);
        keep1 += shfl_xor_f(up2 ? kd[1] : kd[3], 32);
        float sc = (up1 ? keep1 : keep0) + shfl_xor_f(up1 ? keep0 : keep1, 16);
        sc = (base + lane < kv_hi) ? sc * p.scale_log2 : kNegInf;

        const float m_new = fmaxf(m, wave_max(sc));  // finite: key `base` is visible
        const float alpha = fast_exp2(m - m_new);
        const float pr = fast_exp2(sc - m_new);
        lsum = lsum * alpha + pr;
        m = m_new;
#pragma unroll
        for (int k = 0; k < NIV; ++k) acc[k] *= alpha;

        lds_p[lane] = pr;
        wave_lds_sync();
        const bool tail = base + 64 > kv_hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (base + kBlock * j < kv_hi) {
            float pk[X];
#pragma unroll
            for (int e = 0; e < X; e += 4) {
              const f32x4 v4 = *reinterpret_cast<const f32x4*>(&lds_p[kBlock * j + (lane % LPR) * X + e]);
              pk[e] = v4[0]; pk[e + 1] = v4[1]; pk[e + 2] = v4[2]; pk[e + 3] = v4[3];
            }
            // keys past the context may hold anything (even NaN): drop them, not just weight 0
            const int nvis = kv_hi - (base + kBlock * j + (lane % LPR) * X);
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
              float a = acc[k];
#pragma unroll
              for (int e = 0; e < X; ++e) {
                float v;
                if constexpr (kBf16) v = (e & 1) ? bf16_hi(vr[j][k][e >> 1]) : bf16_lo(vr[j][k][e >> 1]);
                else v = __uint_as_float(vr[j][k][e]);
                if (tail && e >= nvis) v = 0.f;
                a = fmaf(pk[e], v, a);
              }
              acc[k] = a;
            }
          }
        }
        wave_lds_sync();
      }
    };
    if (kv_lo < kv_hi) {  // wave-uniform
      if (si.flags & kEntShared) attend(std::false_type{});
      else attend(std::true_type{});
    }
    // finish: l over all lanes, each value column over its LPR lanes
    const float l = wave_sum(lsum);
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
      acc[k] += shfl_xor_f(acc[k], 1);
      if constexpr (LPR == 4) acc[k] += shfl_xor_f(acc[k], 2);
    }
    // every lane of a column group holds the column's value: all of them store it
    if (ex.nps == 0 && w.nparts == 1) {
      T* orow = (T*)p.out + ((int64_t)t * p.Hq + h) * D;
#pragma unroll
      for (int k = 0; k < NIV; ++k) orow[RPI * k + lane / LPR] = Elem<T>::from_f32(acc[k] / l);
    } else {
      float* slot = p.partials + (((int64_t)t * p.Hq + h) * p.maxparts + ex.nps + pidx) * slot_floats(D);
#pragma unroll
      for (int k = 0; k < NIV; ++k) slot[RPI * k + lane / LPR] = acc[k];
      slot[D] = m;
      slot[D + 1] = l;
    }
    if (strided) {
      item += (int)gridDim.x;
    } else {
      __syncthreads();  // every lane has read the previous ticket
      if (threadIdx.x == 0) ticket = atomicAdd(p.ctrl + kValuTicket, 1);
      __syncthreads();
      item = p.valu_resident + wave_uniform(ticket);
    }
  }
}

// ---------------------------------------------------------------- MFMA worker
// One wavefront per item: 16 query rows sharing one KV head x one key
// partition, 32 keys (two pages) per step on v_mfma_f32_16x16x32_bf16, the
// pages of two steps requested before either computes.
//  Scores, transposed: Sᵀ[key][row] = K · Qᵀ with K as the A operand (lane l:
//  key l%16 of the page, 8 head dims per lane, straight from the key page)
//  and Q as the B operand (lane l: row l%16).  The result gives lane l the
//  scores of row l%16 for keys 4(l/16)..+3 of each page.
//  Output, transposed: Oᵀ[dim][row] += Vᵀ · Pᵀ with the value page [D][16]
//  as the A operand (lane l: dim l%16 + 16j, the same 8 keys the lane holds
//  scores for) and Pᵀ (bf16) as the B operand.  Row statistics therefore stay
//  in the lane that owns the row; a row max needs two exchanges (±16, ±32).
//  P enters as a bf16 hi part plus a bf16 lo part (two MFMAs), and the
//  running sum adds exactly those parts, so the result stays a convex
//  combination of the value rows with weights accurate to ~2^-16.
// As in the TILE worker, scores stay unscaled until the exponent (one FMA
// per weight), masks are applied only on steps that reach past the context
// or past a row's position, and a row's exponent reference is raised only
// when its maximum grows by more than kLazyRescale.
// One MFMA tile: the 16 rows of one KV head held by lanes r = lane % 16 (row r at
// token t, query head hh, position pos_r; pos_lo is the tile's lowest position)
// over keys [kv_lo, kv_hi), whose pages the block-table row trow lists.  Leaves
// each lane its row's exponent reference m_r, its share lsum of the row sum and
// the unnormalised output columns 16j + 4(lane/16) .. +3 in oacc[j].
// PIPE: the next step's pages are in flight while a step computes.  That takes
// twice the registers for pages, so the query operand then lives in qs, a
// wavefront-private LDS area of D/32 x 64 entries, and is read back each step.
template <int D, bool PIPE, bool STREAM>
__device__ inline void mfma_tile(const AttnParams& p, int trow, int kvh, int t, int hh, int pos_r, int pos_lo,
                                 int kv_lo, int kv_hi, float& m_r, float& lsum, f32x4 (&oacc)[D / 16],
                                 bf16x8* qs = nullptr) {
  constexpr int KS = D / 32;  // k-steps of the score product
  constexpr int NJ = D / 16;  // 16-dim column blocks of the output
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g4 = lane >> 4;
  const bf16_t* __restrict__ kc = (const bf16_t*)p.k_cache;
  const bf16_t* __restrict__ vc = (const bf16_t*)p.v_cache;
  const int64_t page_elems = (int64_t)kBlock * D;
  const float csc = fmaxf(fabsf(p.scale_log2), 1e-30f);  // scale 0 gives equal weights, as it should
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  if (kv_lo < kv_hi) {
    const int nblk = (kv_hi - kv_lo + kBlock - 1) / kBlock;
    const int bidv = load_block_ids(p, trow, kv_lo / kBlock, nblk, lane);

    bf16x8 qop[KS];
    {
      const bf16_t* qrow = (const bf16_t*)p.q + ((int64_t)t * p.Hq + hh) * D;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const u32x4 qw = ld16(qrow + 32 * k + 8 * g4);
        qop[k] = __builtin_bit_cast(bf16x8, u32x4{qw[0] ^ qflip, qw[1] ^ qflip, qw[2] ^ qflip, qw[3] ^ qflip});
      }
      if constexpr (PIPE) {
#pragma unroll
        for (int k = 0; k < KS; ++k) qs[64 * k + lane] = qop[k];
      }
    }

    // 32 keys (two pages) per step, double-buffered: the next step's pages are
    // requested before the current step computes, so one step's loads are in
    // flight while the other's MFMAs run.  A page past the last one (odd page
    // counts, the partition's tail) reads the last page again: its scores are
    // masked and its values zeroed, and every address stays inside the pool.
    struct Step {
      bf16x8 k0[KS], k1[KS];
      uint32_t vw[NJ][4];  // value operand words: keys 4*g4 + 0..3 of page 0, then of page 1
    };
    auto load = [&](Step& st, int base) {
      const int jb = (base - kv_lo) / kBlock;
      const int64_t pg0 = ((int64_t)readlane(bidv, min(jb, nblk - 1)) * p.Hkv + kvh) * page_elems;
      const int64_t pg1 = ((int64_t)readlane(bidv, min(jb + 1, nblk - 1)) * p.Hkv + kvh) * page_elems;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int off = ((4 * k + g4) * kBlock + r) * 8;
        st.k0[k] = __builtin_bit_cast(bf16x8, ld16_page<STREAM>(kc + pg0 + off));
        st.k1[k] = __builtin_bit_cast(bf16x8, ld16_page<STREAM>(kc + pg1 + off));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int off = (16 * j + r) * kBlock + 4 * g4;
        const u32x2 lo = ld8_page<STREAM>(vc + pg0 + off);
        const u32x2 hi = ld8_page<STREAM>(vc + pg1 + off);
        st.vw[j][0] = lo[0];
        st.vw[j][1] = lo[1];
        st.vw[j][2] = hi[0];
        st.vw[j][3] = hi[1];
      }
    };
    auto compute = [&](Step& st, int base) {
      // unscaled scores of row r for keys base + 16 (e >> 2) + 4 g4 + (e & 3)
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
      // (a compiler-only fence: the query operand is read from LDS here, not kept in registers)
      if constexpr (PIPE) __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const bf16x8 qk = PIPE ? qs[64 * k + lane] : qop[k];
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.k0[k], qk, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(st.k1[k], qk, c1, 0, 0, 0);
      }
      float sc[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = c0[e];
        sc[4 + e] = c1[e];
      }
      if (base + 32 > kv_hi || base + 31 > pos_lo) {  // wave-uniform
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = base + (e >> 2) * kBlock + 4 * g4 + (e & 3);
          sc[e] = (key < kv_hi && key <= pos_r) ? sc[e] : kNegInf;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      mx = max_over_rows(mx);
      const float mloc = mx * csc;  // -inf stays -inf (csc > 0)
      if (__builtin_amdgcn_ballot_w64(mloc > m_r + kLazyRescale)) {
        const float m_new = fmaxf(m_r, mloc);
        const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_r - m_new);
        lsum *= alpha;
#pragma unroll
        for (int j = 0; j < NJ; ++j) oacc[j] *= alpha;
        m_r = m_new;
      }
      const float nmu = m_r == kNegInf ? 0.f : -m_r;  // a row that sees no key yet has weights 0
      uint32_t phw[4], plw[4];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = fast_exp2(fmaf(sc[e], csc, nmu));
        const float p1 = fast_exp2(fmaf(sc[e + 1], csc, nmu));
        const uint32_t hw = pack_bf16x2(p0, p1);
        phw[e >> 1] = hw;
        plw[e >> 1] = pack_bf16x2(p0 - bf16_lo(hw), p1 - bf16_hi(hw));
        psum += p0 + p1;
      }
      const bf16x8 pop_hi = __builtin_bit_cast(bf16x8, u32x4{phw[0], phw[1], phw[2], phw[3]});
      const bf16x8 pop_lo = __builtin_bit_cast(bf16x8, u32x4{plw[0], plw[1], plw[2], plw[3]});
      lsum += psum;
      if (base + 32 > kv_hi) {
        // keys past kv_hi may hold anything (even NaN): zero them in the value operand
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = base + (e >> 2) * kBlock + 4 * g4 + (e & 3);
          const uint32_t keep = key < kv_hi ? 0xffffffffu : (e & 1) ? 0x0000ffffu : 0xffff0000u;  // a select
#pragma unroll
          for (int j = 0; j < NJ; ++j) st.vw[j][e >> 1] &= keep;
        }
      }
      // the high parts first, then the low parts: no MFMA waits on the one before it
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{st.vw[j][0], st.vw[j][1], st.vw[j][2], st.vw[j][3]});
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_hi, oacc[j], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{st.vw[j][0], st.vw[j][1], st.vw[j][2], st.vw[j][3]});
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_lo, oacc[j], 0, 0, 0);
      }
    };
    Step sa, sb;
    if constexpr (PIPE) {
      // Two register sets in turn (unrolled by two: no copies between them);
      // the loop conditions are wave-uniform.  The scheduling barriers keep
      // the next step's loads ahead of the current step's arithmetic.
      load(sa, kv_lo);
      for (int base = kv_lo;; base += 64) {
        if (base + 32 >= kv_hi) {
          compute(sa, base);
          break;
        }
        load(sb, base + 32);
        __builtin_amdgcn_sched_barrier(0);
        compute(sa, base);
        if (base + 64 >= kv_hi) {
          compute(sb, base + 32);
          break;
        }
        load(sa, base + 64);
        __builtin_amdgcn_sched_barrier(0);
        compute(sb, base + 32);
      }
    } else {
      // 64 keys requested, then computed: half the registers of the pipelined loop
      for (int base = kv_lo; base < kv_hi; base += 64) {
        load(sa, base);
        load(sb, base + 32);
        compute(sa, base);
        if (base + 32 < kv_hi) compute(sb, base + 32);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void mfma_attn_kernel(AttnParams p) {
  constexpr int NJ = D / 16;  // 16-dim column blocks of the output
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g4 = lane >> 4;
  const int wave_id = wave_uniform((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int nwaves = (int)gridDim.x * 4;
  const int total = wave_uniform(p.ctrl[3]);
  if ((int)blockIdx.x * 4 >= total) return;  // no wavefront of this workgroup has an item
  __shared__ int skip[kSkip];
  const SkipTable tab = stage_skip(skip, p.pre_m, p.num_ent);

  for (int item = wave_id; item < total; item += nwaves) {
    const SeqHit hit = find_seq(skip, tab, p.pre_m, p.num_ent, item);
    const int s = hit.s;
    const int local = item - hit.first;
    const SeqInfo si = seq_record(p, s);
    const EntX ex = ent_x(p, s, si.flags);
    const bool grp = si.flags & kEntGroup;  // rows of several members over their shared keys
    const SeqWork w = grp ? group_work(p.Hkv, si.L) : seq_work(false, p.G, p.Hq, p.Hkv, si.q_len, si.L - ex.koff);
    const int pidx = local % w.nparts;
    const int rest = local / w.nparts;
    const int kvh = rest % p.Hkv;
    const int tile = rest / p.Hkv;
    const int rows_total = si.q_len * p.G;
    // Rows past the sequence's last row (the padding of the last tile) repeat
    // that last row: they compute its values and store the same bytes to its
    // address, so no lane ever needs a branch or a dummy destination.
    const int R = min(tile * kTileRows + r, rows_total - 1);
    const int qi = R / p.G;
    const int hh = kvh * p.G + R % p.G;
    const int t = si.a + qi;
    const int pos_r = grp ? si.L - 1 : si.L - si.q_len + qi;
    const int last_row = min(tile * kTileRows + kTileRows - 1, rows_total - 1);
    const int tile_pos_max = grp ? si.L - 1 : si.L - si.q_len + last_row / p.G;
    const int kv_lo = ex.koff + pidx * w.part;
    const int kv_hi = min(kv_lo + w.part, tile_pos_max + 1);

    float m_r = kNegInf, lsum = 0.f;
    f32x4 oacc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int pos_lo = grp ? si.L - 1 : si.L - si.q_len + (tile * kTileRows) / p.G;  // lowest row position
    // a group reads its first member's table
    if (!grp && (si.flags & kEntShared))  // wave-uniform; a group's shared pages are read once
      mfma_tile<D, false, false>(p, ex.trow, kvh, t, hh, pos_r, pos_lo, kv_lo, kv_hi, m_r, lsum, oacc);
    else
      mfma_tile<D, false, true>(p, ex.trow, kvh, t, hh, pos_r, pos_lo, kv_lo, kv_hi, m_r, lsum, oacc);
    const float l = sum_over_rows(lsum);
    if (!grp && ex.nps == 0 && w.nparts == 1) {
      bf16_t* orow = (bf16_t*)p.out + ((int64_t)t * p.Hq + hh) * D;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x2 pk = {pack_bf16x2(oacc[j][0] / l, oacc[j][1] / l), pack_bf16x2(oacc[j][2] / l, oacc[j][3] / l)};
        *reinterpret_cast<u32x2*>(orow + 16 * j + 4 * g4) = pk;
      }
    } else {
      float* slot = p.partials + (((int64_t)t * p.Hq + hh) * p.maxparts + ex.nps + pidx) * slot_floats(D);
#pragma unroll
      for (int j = 0; j < NJ; ++j) *reinterpret_cast<f32x4*>(slot + 16 * j + 4 * g4) = oacc[j];
      slot[D] = m_r;  // the four lanes of a row hold the same m and l
      slot[D + 1] = l;
    }
  }
}

// ---------------------------------------------------------------- one-pass GQA decode
// Batches whose every row is a single-position decode, with 2..16 query heads
// per KV head (the MFMA worker's GQA rows), skip the planner and the merge
// kernel.  One workgroup of kDecWaves wavefronts takes a chunk of
// kDecWaves x kDecPart keys of one (sequence, KV head): wavefront w
// computes partition w of the chunk as an MFMA tile (rows = the G query heads),
// and the chunk's partial states are merged through LDS ("第 15 章" §15.1
// rescaling applied to finished states).  A context of one chunk writes its
// output directly.  A longer context writes one state per chunk; the
// workgroup that completes the last chunk of its (sequence, KV head) merges
// them.  It knows it is last from a completion counter in the workspace: a
// 64-bit word whose high half holds a tag of the call and whose low half
// counts the chunks done; a word whose tag is not this call's counts as zero,
// and the merging workgroup leaves (tag, 0) behind, so neither an
// uninitialised workspace nor a replay of a captured call with the same tag
// sees stale counts.  Items come from the host-known bounds only (no sequence
// is read by the host): workgroup (s, kvh, chunk) exits at once when the
// chunk lies past the sequence's context.
constexpr int kDecWaves = 8;
// Keys per wavefront: one fixed length, so a sequence's partitions (and its
// result) never depend on the rest of the batch.  256 keys keep each
// wavefront streaming long enough to amortise its start (sequence record,
// block table, query rows) and its share of the chunk merge.
constexpr int kDecPart = kPartMfmaDecode;
__host__ __device__ constexpr int dec_chunks(int L) { return (L + kDecWaves * kDecPart - 1) / (kDecWaves * kDecPart); }

__device__ inline uint32_t dec_tagged_count(unsigned long long* ctr, uint32_t tag) {
  // one thread: counts this chunk; returns the number of chunks done including it
  unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if ((uint32_t)(old >> 32) == tag) return (uint32_t)atomicAdd(ctr, 1ull) + 1u;
    const unsigned long long want = ((unsigned long long)tag << 32) | 1ull;
    const unsigned long long got = atomicCAS(ctr, old, want);
    if (got == old) return 1u;
    old = got;
  }
}

template <int D>
__global__ __launch_bounds__(64 * kDecWaves, 1) void gqa_decode_kernel(AttnParams p) {
  constexpr int NJ = D / 16;
  constexpr int SF = slot_floats(D);
  // one state per wavefront and row: O[D], m, l
  __shared__ float st_lds[kDecWaves][kTileRows][D + 2];
  __shared__ bf16x8 q_lds[kDecWaves][D / 32 * 64];  // each wavefront's query operand
  __shared__ int flag;
  const int lane = threadIdx.x & 63;
  const int wv = wave_uniform((int)(threadIdx.x >> 6));
  const int r = lane & 15, g4 = lane >> 4;
  const int nchunk_bound = max(1, dec_chunks(p.max_ctx));  // dec_chunks grows with L
  const int item = (int)blockIdx.x;
  const int chunk = item % nchunk_bound;
  const int s = item / nchunk_bound / p.Hkv;
  const int kvh = item / nchunk_bound % p.Hkv;
  if (item == 0 && threadIdx.x == 0 && (p.qsl[0] != 0 || p.qsl[p.num_seqs] != p.T))
    flag_status(p.dev_status, PA_DEV_BAD_LENGTH);
  SeqInfo si = read_seq(p, s);
  si.a = wave_uniform(si.a);
  si.q_len = wave_uniform(si.q_len);
  si.L = wave_uniform(si.L);
  const bool ok = wave_uniform((int)si.ok) != 0;
  if (!ok) {
    if (chunk == 0 && kvh == 0 && threadIdx.x == 0) flag_status(p.dev_status, PA_DEV_BAD_LENGTH);
    return;
  }
  const int part = kDecPart;
  const int nchunks = dec_chunks(si.L);
  if (si.q_len == 0 || chunk >= nchunks) return;  // workgroup-uniform
  const int t = si.a;
  const int G = p.G;
  const int R = min(r, G - 1);  // rows past the last query head repeat it
  const int hh = kvh * G + R;
  const int pos = si.L - 1;
  const int kv_lo = (chunk * kDecWaves + wv) * part;
  const int kv_hi = min(kv_lo + part, si.L);

  float m_r = kNegInf, lsum = 0.f;
  f32x4 oacc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // pages shared with a neighbouring sequence (forks of one prompt) are loaded plain
  const int32_t first_blk = p.block_tables[(int64_t)s * p.mbps];
  const bool shared = (s > 0 && p.context_lens[s - 1] > 0 && p.block_tables[(int64_t)(s - 1) * p.mbps] == first_blk) ||
                      (s + 1 < p.num_seqs && p.context_lens[s + 1] > 0 &&
                       p.block_tables[(int64_t)(s + 1) * p.mbps] == first_blk);
  if (kv_lo < kv_hi) {  // wave-uniform
    if (wave_uniform((int)shared))
      mfma_tile<D, true, false>(p, s, kvh, t, hh, pos, pos, kv_lo, kv_hi, m_r, lsum, oacc, q_lds[wv]);
    else
      mfma_tile<D, true, true>(p, s, kvh, t, hh, pos, pos, kv_lo, kv_hi, m_r, lsum, oacc, q_lds[wv]);
  }
  const float l = sum_over_rows(lsum);
  // every lane of a row stores the same m and l; each lane its own columns
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) st_lds[wv][r][16 * j + 4 * g4 + e] = oacc[j][e];
  st_lds[wv][r][D] = m_r;
  st_lds[wv][r][D + 1] = l;
  __syncthreads();

  // merge the chunk's partitions: wavefront w takes rows w, w + kDecWaves, ...; lane c has
  // columns 2c, 2c + 1 (D = 128) or column c (D = 64)
  constexpr int CPL = D / 64;  // columns per lane
  const bool single = nchunks == 1;
  for (int row = wv; row < G; row += kDecWaves) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, st_lds[w][row][D]);
    float lt = 0.f, o[CPL] = {};
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = st_lds[w][row][D];
      const float wt = fast_exp2(mw == kNegInf ? kNegInf : mw - M);  // an empty partition weighs 0
      lt = fmaf(st_lds[w][row][D + 1], wt, lt);
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] = fmaf(st_lds[w][row][CPL * lane + c], wt, o[c]);
    }
    const int hrow = kvh * G + row;
    if (single) {
      bf16_t* orow = (bf16_t*)p.out + ((int64_t)t * p.Hq + hrow) * D;
#pragma unroll
      for (int c = 0; c < CPL; ++c) orow[CPL * lane + c] = Elem<bf16_t>::from_f32(o[c] / lt);
    } else {
      // read back within this dispatch, possibly on another XCD: agent-scope stores
      float* slot = p.partials + (((int64_t)t * p.Hq + hrow) * p.maxparts + chunk) * SF;
#pragma unroll
      for (int c = 0; c < CPL; ++c) st_agent(slot + CPL * lane + c, o[c]);
      if (lane == 0) {
        st_agent(slot + D, M);
        st_agent(slot + D + 1, lt);
      }
    }
  }
  if (single) return;

  // the workgroup that completes the last chunk merges the chunk states
  wait_stores();  // this workgroup's chunk states are visible before it is counted
  __syncthreads();
  unsigned long long* ctr = p.dec_ctr + (int64_t)s * p.Hkv + kvh;
  if (threadIdx.x == 0) flag = (int)dec_tagged_count(ctr, p.call_tag);
  __syncthreads();
  if (wave_uniform(flag) != nchunks) return;
  // Reached only after every chunk was counted, and each workgroup counted its chunk once
  // its agent-scope stores were acknowledged: agent-scope loads see them all.
  // One row per wavefront at a time, 32 chunks per round (an online-softmax merge across
  // rounds): lane c%32 loads chunk c's m and l, half-wavefront h loads the outputs of
  // chunks h, h + 2, ..., lane l%32 holding columns l%32 + 32q (q < D/32).  Every load of
  // a round is issued before any is used, so a round costs one memory round trip.
  constexpr int CPH = D / 32;  // columns per lane
  constexpr int RC = 32;       // chunks per round
  const int half = lane >> 5, cl = lane & 31;
  for (int row = wv; row < G; row += kDecWaves) {
    const int hrow = kvh * G + row;
    const float* base = p.partials + ((int64_t)t * p.Hq + hrow) * p.maxparts * SF;
    float M = kNegInf, lt = 0.f, o[CPH] = {};
    for (int c0 = 0; c0 < nchunks; c0 += RC) {
      const int n = min(RC, nchunks - c0);
      const float* sm = base + (int64_t)(c0 + min(cl, n - 1)) * SF + D;
      const float mraw = ld_agent(sm), lc = ld_agent(sm + 1);
      float v[RC / 2][CPH];
#pragma unroll
      for (int i = 0; i < RC / 2; ++i) {
        const float* sk = base + (int64_t)(c0 + min(half + 2 * i, n - 1)) * SF + cl;
#pragma unroll
        for (int q = 0; q < CPH; ++q) v[i][q] = ld_agent(sk + 32 * q);
      }
      const float mc = cl < n ? mraw : kNegInf;
      const float Mn = fmaxf(M, wave_max(mc));
      const float keep = M == kNegInf ? 0.f : fast_exp2(M - Mn);  // rescales the earlier rounds
      const float wc = mc == kNegInf ? 0.f : fast_exp2(mc - Mn);   // a state with no finite score weighs 0
      lt = fmaf(lt, keep, half == 0 ? lc * wc : 0.f);
#pragma unroll
      for (int q = 0; q < CPH; ++q) o[q] *= keep;
#pragma unroll
      for (int i = 0; i < RC / 2; ++i) {
        const float wk = __shfl(wc, half + 2 * i, kWave);  // 0 for chunks past n
#pragma unroll
        for (int q = 0; q < CPH; ++q) o[q] = fmaf(v[i][q], wk, o[q]);
      }
      M = Mn;
    }
    lt = wave_sum(lt);
#pragma unroll
    for (int q = 0; q < CPH; ++q) o[q] += __shfl_xor(o[q], 32, kWave);
    if (half == 0) {
      bf16_t* orow = (bf16_t*)p.out + ((int64_t)t * p.Hq + hrow) * D + cl;
#pragma unroll
      for (int q = 0; q < CPH; ++q) orow[32 * q] = Elem<bf16_t>::from_f32(o[q] / lt);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0)  // the next call with this tag starts at zero
    __hip_atomic_store(ctr, (unsigned long long)p.call_tag << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- TILE worker
// One workgroup of kTileWaves wavefronts per item: kBigRows query rows sharing
// one KV head x one key partition; wavefront w owns rows 32w .. 32w+31 of the
// item.  Every product is a 32x32x16 MFMA (v_mfma_f32_32x32x16_*):
//  Scores, transposed: Sᵀ[key][row] = K · Qᵀ, 32 keys x 32 rows per MFMA,
//  D/16 MFMAs over the head dimension.  Lane l holds row l%32 and, in
//  accumulator j, key 16(j/8) + 8(l/32) + j%8 of the 32-key step: the key
//  operand's rows are loaded in a permuted order (bits 2 and 3 of the key
//  index swapped) so that each lane ends with 8 consecutive keys per 16-key
//  block, which is the layout P·V needs for its B operand, with no exchange.
//  Output, transposed: Oᵀ[dim][row] += Vᵀ · Pᵀ, 32 dims x 32 rows x 16 keys
//  per MFMA; the value operand of lane l is 8 consecutive keys of dim l%32,
//  i.e. one 16-byte piece of a value page [D][16].
// Each lane's row statistics: the two lane halves l, l+32 hold the same row
// for different keys, so a row max is a 16-value max and one lane swap.
// Steps of 32 keys: all operands of a step (8 KiB of keys, 8 KiB of values at
// D = 128) are staged in LDS in the order the lanes read them (piece 64b + l is
// lane l's operand of block b), so every operand read is 64 consecutive
// 16-byte pieces.  Every wavefront loads two 1 KiB blocks of each step, three
// steps ahead into one of two register sets, and stores them two steps ahead
// into a four-stage ring; one barrier per two steps publishes the two stages
// stored since the last one and frees the two read before it.  The 256 rows of
// an item share every key and value piece it reads from HBM (or L2).
// Softmax ("第 15 章" §15.1 recurrence): scores stay unscaled until the
// exponent (p = 2^(s·c − m) with c = |scale|·log2 e, one FMA; a negative scale
// flips the sign bits of q instead, which is exact).  A row's reference m is
// its maximum over the item's first step (every row that sees a key of the
// item sees its first key; O and l share the reference, so O / l does not
// depend on it), and the other steps compute their weights against it with
// no row maximum.
// P·V precision: the weights enter the half-precision MFMA as p rounded to
// half (relative error 2^-11; weights more than 2^14 below the first step's
// maximum become subnormal, an absolute error of at most 2^-25 against a
// weight of 1), the values as half, converted once per workgroup when they
// are stored to LDS (exact for bfloat16 values of magnitude below 2^16 down
// to 2^-17); the row sum adds exactly the rounded weights (v_dot2_f32_f16).
// A weight of 65520 or more (a row maximum that grew by 16 or more in log2
// after the first step) or a bfloat16 value of magnitude 65520 or more
// becomes an infinite half, and the output of every row that uses it becomes
// infinite or NaN (0 x inf); the wavefronts check their outputs once after
// the last step, and an item with a non-finite one is computed again with
// the values left in bfloat16, the row maximum on every step (the reference
// raised when it grew by more than kLazyRescale), and the weights split into
// a bfloat16 high and low part (two MFMAs, weights exact to about 2^-16),
// which holds for every finite input.
// Work distribution: items are numbered so that the row tiles of one (KV
// head, partition) are consecutive; the item list is cut into eight equal
// slices, one per XCD (each XCD has its own L2), and the workgroups of an XCD
// take tickets from their slice first, then from the other slices in turn.
// Row tiles sharing keys and values therefore run at about the same time on
// one L2, which serves the second read.  One atomic per item, by one thread
// between two barriers: the one per-lane branch of the worker.
template <int D>
struct TileShape {
  static constexpr int KB = D / 16;           // key operand blocks per step (one per score MFMA)
  static constexpr int DB = D / 32;           // 32-dim blocks of the output
  static constexpr int VB = 2 * DB;           // value operand blocks per step: dim block x 16-key block
  static constexpr int NB = KB + VB;          // 1 KiB operand blocks per step
  static constexpr int BPW = NB / kTileWaves; // blocks each wavefront loads per step
  static_assert(NB % kTileWaves == 0 && BPW >= 1, "the blocks of a step split evenly over the wavefronts");
};

// Marks a rarely taken, wave-uniform branch that must stay a branch: the
// compiler would otherwise run its body on every pass with neutral values
// (for example multiply the output by a rescale factor of 1), which costs more
// than the branch.  An empty volatile asm cannot be executed speculatively.
__device__ inline void keep_branch() { asm volatile(""); }


template <int D>
__global__ __launch_bounds__(64 * kTileWaves, 1) void tile_attn_kernel(AttnParams p) {
  using TS = TileShape<D>;
  constexpr int KB = TS::KB, DB = TS::DB, NB = TS::NB, BPW = TS::BPW;
  static_assert(kPartTile % 32 == 0 && kPartTile <= 64 * kBlock, "a partition is whole steps of at most 64 pages");
  __shared__ u32x4 stage[kTileStages][NB * 64];
  __shared__ int skip[kSkip];
  __shared__ int ticket;
  __shared__ int wave_flag[kTileWaves];

  const int lane = threadIdx.x & 63;
  const int wv = wave_uniform((int)(threadIdx.x >> 6));
  const int n = lane & 31, h = lane >> 5;
  const int total = wave_uniform(p.ctrl[4]);
  const bf16_t* __restrict__ kc = (const bf16_t*)p.k_cache;
  const bf16_t* __restrict__ vc = (const bf16_t*)p.v_cache;
  const int blk_elems = p.Hkv * kBlock * D;  // elements of one physical block (all KV heads), below 2^31
  const float csc = fmaxf(fabsf(p.scale_log2), 1e-30f);  // scale 0 gives equal weights, as it should
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  const SkipTable tab = stage_skip(skip, p.pre_t, p.num_ent);
  const int xcc = wave_uniform(__builtin_amdgcn_s_getreg(kHwRegXccId) & (kXcds - 1));

  // Next item: from this XCD's slice, then the following slices in turn; -1 when all are done.
  // The items are dealt to the slices in chunks of four (slice x holds chunks x, x + 8, ...),
  // so each slice holds an even share of every sequence's items, in their order (partition-
  // major, the short last partitions last), and the row tiles of one (KV head, partition),
  // consecutive items, mostly fall in one chunk and so share an XCD's L2.
  int qi = 0;
  auto next_item = [&]() {
#pragma clang loop unroll(disable)
    while (qi < kXcds) {
      const int qq = (xcc + qi) & (kXcds - 1);
      __syncthreads();  // every thread has read the previous ticket (and is done with the stages)
      if (threadIdx.x == 0) ticket = atomicAdd(p.ctrl + 8 + qq, 1);
      __syncthreads();
      const int t = wave_uniform(ticket);
      const int64_t item = (((int64_t)(t >> 2) * kXcds + qq) << 2) + (t & 3);
      if (item < total) return (int)item;
      ++qi;
    }
    return -1;
  };

  for (;;) {
    const int item = next_item();
    if (item < 0) break;
    const SeqHit hit = find_seq(skip, tab, p.pre_t, p.num_ent, item);
    const int s = hit.s;
    const int local = item - hit.first;
    const SeqInfo si = seq_record(p, s);
    const SeqWork w = seq_work(false, p.G, p.Hq, p.Hkv, si.q_len, si.L);
    const int rows_total = si.q_len * p.G;
    const int ntiles = (rows_total + kBigRows - 1) / kBigRows;
    // partition-major: row tiles of one (KV head, partition) are consecutive items, then the
    // KV heads, then the partitions (the short last partition of a sequence comes last)
    const int tile = local % ntiles;
    const int rest = local / ntiles;
    const int kvh = rest % p.Hkv;
    const int pidx = rest / p.Hkv;
    const int first = si.L - si.q_len;  // position of query row 0
    const int tile_last = min(tile * kBigRows + kBigRows - 1, rows_total - 1);
    const int kv_lo = pidx * w.part;
    const int kv_hi = min(kv_lo + w.part, first + tile_last / p.G + 1);
    if (kv_lo >= kv_hi) continue;  // no row of the tile sees this partition: the merge skips it

    // this wavefront's rows; padding rows repeat the last row (they store the same bytes to its address)
    const int row0 = tile * kBigRows + 32 * wv;
    const bool active = row0 < rows_total;
    const int w_pos_lo = first + min(row0, rows_total - 1) / p.G;
    const int w_kv_hi = active ? min(kv_hi, first + min(row0 + 31, rows_total - 1) / p.G + 1) : kv_lo;
    const int R = min(row0 + n, rows_total - 1);
    const int hh = kvh * p.G + R % p.G;
    const int tok = si.a + R / p.G;
    const int pos_r = first + R / p.G;
    bf16x8 qop[KB];
    {
      const bf16_t* qrow = (const bf16_t*)p.q + ((int64_t)tok * p.Hq + hh) * D;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const u32x4 qw = ld16(qrow + 16 * kk + 8 * h);
        qop[kk] = __builtin_bit_cast(bf16x8, u32x4{qw[0] ^ qflip, qw[1] ^ qflip, qw[2] ^ qflip, qw[3] ^ qflip});
      }
    }

    const int nblk = (kv_hi - kv_lo + kBlock - 1) / kBlock;
    const int bidv = load_block_ids(p, s, kv_lo / kBlock, nblk, lane);
    const int nsteps = (kv_hi - kv_lo + 31) / 32;
    const int nw = (w_kv_hi - kv_lo + 31) / 32;  // steps this wavefront computes (a prefix of the item's)
    const int head_off = kvh * kBlock * D;  // element offset of the KV head inside a block (below 2^31)

    // The blocks this wavefront loads: block b = wv + kTileWaves u; b < KB is key block b
    // (lane l: key of in-step index π(l%32) with bits 2 and 3 swapped, dims 16b + 8(l/32) ..),
    // else value block b - KB = 2 db + kb (lane l: dim 32 db + l%32, keys 16 kb + 8(l/32) ..).
    uint32_t loff[BPW];
    bool second_page[BPW];
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int b = wv + kTileWaves * u;
      // element offset inside the block's (physical block, KV head) page run, KV head included
      if (b < KB) {
        const int kp = 8 * ((n >> 2) & 1) + 4 * ((n >> 3) & 1) + (n & 3);
        loff[u] = (uint32_t)(head_off + ((2 * b + h) * kBlock + kp) * 8);
        second_page[u] = n >= 16;
      } else {
        const int vb = b - KB;
        loff[u] = (uint32_t)(head_off + (32 * (vb >> 1) + n) * kBlock + 8 * h);
        second_page[u] = (vb & 1) != 0;
      }
    }
    auto fetch = [&](int st, u32x4 (&reg)[BPW]) {
      const int64_t pg0 = (int64_t)readlane(bidv, min(2 * st, nblk - 1)) * (int64_t)blk_elems;
      const int64_t pg1 = (int64_t)readlane(bidv, min(2 * st + 1, nblk - 1)) * (int64_t)blk_elems;
#pragma unroll
      for (int u = 0; u < BPW; ++u) {
        const bool key = wv + kTileWaves * u < KB;  // wave-uniform
        reg[u] = ld16((key ? kc : vc) + (second_page[u] ? pg1 : pg0) + loff[u]);
      }
    };

    auto pass = [&](auto exact_tag) {
      constexpr bool kExact = decltype(exact_tag)::value;
      bool nonfinite = false;
      // Stage step st: keys as loaded; values zeroed past kv_hi (the pool there may hold
      // anything), then converted to half unless kExact (a magnitude of 65520 or more
      // becomes an infinite half, which makes the output of every row that uses it
      // non-finite: checked once per item, after the last step).
      auto put = [&](u32x4 (&reg)[BPW], int st) {
        u32x4* img = stage[st % kTileStages];
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
          const int b = wv + kTileWaves * u;
          u32x4 v = reg[u];
          if (b >= KB) {
            if (kv_lo + 32 * st + 32 > kv_hi) {  // wave-uniform: the step reaches past the partition
              const int kfirst = kv_lo + 32 * st + 16 * ((b - KB) & 1) + 8 * h;  // key of the piece's first value
#pragma unroll
              for (int e = 0; e < 4; ++e)
                v[e] &= (kfirst + 2 * e < kv_hi ? 0x0000ffffu : 0u) | (kfirst + 2 * e + 1 < kv_hi ? 0xffff0000u : 0u);
            }
            if constexpr (!kExact) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = pack_f16x2(bf16_lo(v[e]), bf16_hi(v[e]));
            }
          }
          img[b * 64 + lane] = v;
        }
      };

      float m_used = kNegInf, lsum = 0.f;
      float nmu = 0.f;  // exponent offset: -m_used (0 while m_used is -inf: those rows' weights are 0)
      f32x16 oacc[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;

      auto scores = [&](int st, f32x16& c) {
        const u32x4* img = stage[st % kTileStages];
#pragma unroll
        for (int j = 0; j < 16; ++j) c[j] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, img[kk * 64 + lane]), qop[kk], c, 0,
                                                      0, 0);
      };

      // Raises each row's reference to the row's maximum when that grew past it by more
      // than kLazyRescale (the branch is taken when any row of the wavefront needs it).
      auto raise_reference = [&](const float (&sc)[16]) {
        // the scores pass through an empty asm so that the maximum is computed here, not
        // hoisted in front of the branches that lead here
        float t[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          t[j] = sc[j];
          asm volatile("" : "+v"(t[j]));
        }
        float mx = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(t[8], t[9]), fmaxf(t[10], t[11])),
                             fmaxf(fmaxf(t[12], t[13]), fmaxf(t[14], t[15]))));
        {
          typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
          const u32x2v sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mloc = mx * csc;  // -inf stays -inf (csc > 0)
        if (__builtin_amdgcn_ballot_w64(mloc > m_used + kLazyRescale)) {
          keep_branch();
          const float m_new = fmaxf(m_used, mloc);
          const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_used - m_new);
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          m_used = m_new;
          nmu = m_used == kNegInf ? 0.f : -m_used;
        }
      };

      // softmax of step st (scores in c) and its P·V
      auto softmax_pv = [&](int st, f32x16& c) {
        const int kbase = kv_lo + 32 * st;
        float sc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[j] = c[j];
        if (kbase + 31 > w_pos_lo || kbase + 32 > kv_hi) {  // some key lies past some row's position or the partition
          keep_branch();
          // in-step key 16(j/8) + 8h + j%8 is visible iff it is <= lim
          const int lim = min(kv_hi - 1, pos_r) - kbase - 8 * h;
#pragma unroll
          for (int j = 0; j < 16; ++j) sc[j] = 16 * (j >> 3) + (j & 7) <= lim ? sc[j] : kNegInf;
        }
        const u32x4* img = stage[st % kTileStages];
        if constexpr (!kExact) {
          // The reference is the rows' maximum over the first step (every row that sees a
          // key of the item sees key kv_lo) and stays fixed for the item: no row maximum on
          // the other steps.  A weight p of 65520 or more (the maximum grew by 16 or more
          // in log2) rounds to an infinite half and makes the row's output non-finite,
          // which the check after the last step catches.
          if (st == 0) {
            keep_branch();
            raise_reference(sc);
          }
          f16x8 pw[2];
          const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w4[e] = pack_f16x2(fast_exp2(fmaf(sc[8 * kb + 2 * e], csc, nmu)),
                                 fast_exp2(fmaf(sc[8 * kb + 2 * e + 1], csc, nmu)));
              lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w4[e]), ones, lsum, false);
            }
            pw[kb] = __builtin_bit_cast(f16x8, u32x4{w4[0], w4[1], w4[2], w4[3]});
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, img[(KB + 2 * db + kb) * 64 + lane]), pw[kb], oacc[db], 0, 0, 0);
        } else {
          raise_reference(sc);
          bf16x8 phi[2], plo[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = fast_exp2(fmaf(sc[8 * kb + 2 * e], csc, nmu));
              const float p1 = fast_exp2(fmaf(sc[8 * kb + 2 * e + 1], csc, nmu));
              hw[e] = pack_bf16x2(p0, p1);
              lw[e] = pack_bf16x2(p0 - bf16_lo(hw[e]), p1 - bf16_hi(hw[e]));
              lsum += p0 + p1;
            }
            phi[kb] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
            plo[kb] = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const bf16x8 va = __builtin_bit_cast(bf16x8, img[(KB + 2 * db + kb) * 64 + lane]);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, phi[kb], oacc[db], 0, 0, 0);
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, plo[kb], oacc[db], 0, 0, 0);
            }
        }
      };

      // One step of the loop, unrolled by two so that each register set stays in fixed
      // registers: set rs_put holds step st+2 (stored at the end), set rs_fetch receives
      // step st+3.  Fetches past the last step read the last step again, so the number of
      // loads in flight is the same on every path.  One barrier per two steps: the one
      // before an even step st publishes stages st and st+1 (stored in steps st-2 and
      // st-1) and frees stages st-2 and st-1, which steps st and st+1 overwrite with st+2
      // and st+3 (a ring of four stages).
      auto step = [&](int st, u32x4 (&rs_fetch)[BPW], u32x4 (&rs_put)[BPW]) {
        if ((st & 1) == 0) __syncthreads();
        fetch(min(st + 3, nsteps - 1), rs_fetch);
        if (st < nw) {
          f32x16 c;
          scores(st, c);
          softmax_pv(st, c);
        }
        put(rs_put, st + 2);
      };

      u32x4 rset0[BPW], rset1[BPW];
      __syncthreads();  // every wavefront is done with the stages of the previous item (or pass)
      fetch(0, rset0);
      fetch(min(1, nsteps - 1), rset1);
      put(rset0, 0);
      fetch(min(2, nsteps - 1), rset0);
      put(rset1, 1);
      __syncthreads();
      int st = 0;
      for (; st + 2 <= nsteps; st += 2) {
        step(st, rset1, rset0);
        step(st + 1, rset0, rset1);
      }
      if (st < nsteps) step(st, rset1, rset0);

      if constexpr (!kExact) {
        // an infinite half weight or value reaches the output as inf or NaN (0 x inf);
        // otherwise every partial sum is finite (p < 2^16 and |v| < 2^16 over at most 1024 keys)
        float all = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) all += oacc[db][j];
        // an integer test of the exponent bits, kept opaque: built without NaNs, the compiler
        // would otherwise fold it into a float compare with infinity, which a NaN fails
        uint32_t bits = __float_as_uint(all);
        asm volatile("" : "+v"(bits));
        nonfinite = (bits & 0x7f800000u) == 0x7f800000u;
      }
      if (active) {
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        const u32x2v sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // the row's two lane halves
        if (w.nparts == 1) {
          bf16_t* orow = (bf16_t*)p.out + ((int64_t)tok * p.Hq + hh) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const u32x2 pk = {pack_bf16x2(oacc[db][4 * i] / l, oacc[db][4 * i + 1] / l),
                                pack_bf16x2(oacc[db][4 * i + 2] / l, oacc[db][4 * i + 3] / l)};
              *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * i + 4 * h) = pk;
            }
        } else {
          float* slot = p.partials + (((int64_t)tok * p.Hq + hh) * p.maxparts + pidx) * slot_floats(D);
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              *reinterpret_cast<f32x4*>(slot + 32 * db + 8 * i + 4 * h) =
                  f32x4{oacc[db][4 * i], oacc[db][4 * i + 1], oacc[db][4 * i + 2], oacc[db][4 * i + 3]};
          slot[D] = m_used;
          slot[D + 1] = l;
        }
      }
      return nonfinite;
    };

    const bool oor = pass(std::false_type{});
    wave_flag[wv] = __builtin_amdgcn_ballot_w64(oor) != 0 ? 1 : 0;  // every lane writes the wave's value
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int k = 0; k < kTileWaves; ++k) any |= wave_flag[k];
    if (wave_uniform(any)) pass(std::true_type{});
  }
}

// ---------------------------------------------------------------- merge
// Persistent workgroups walk the planner's list of (query token, query head)
// rows whose context was split, WPR wavefronts per row.  A
// lane covers four output columns of one partition, so one 16-byte load per
// lane reads 64 / (D / 4) partitions at once, and each lane keeps U loads in
// flight; the WPR wavefronts of a workgroup take interleaved shares of the
// partitions and add their sums through LDS.  Weights: M = max_p m_p,
// l = Σ_p l_p 2^(m_p − M), out = Σ_p O_p 2^(m_p − M) / l.
template <typename T, int D, int WPR>
__global__ __launch_bounds__(256) void merge_kernel(AttnParams p) {
  constexpr int LPP = D / 4;     // lanes per partition
  constexpr int PPI = 64 / LPP;  // partitions per wavefront load
  constexpr int U = 4;           // loads in flight per lane
  constexpr int RPB = 4 / WPR;   // rows merged at once per workgroup
  constexpr int SF = slot_floats(D);
  __shared__ f32x4 red[4][64];
  __shared__ int skip[kSkip];
  const int lane = threadIdx.x & 63;
  const int wv = wave_uniform((int)(threadIdx.x >> 6));
  const int sub = wv % WPR;
  const int total = wave_uniform(p.ctrl[5]);
  const SkipTable tab = stage_skip(skip, p.pre_g, p.num_ent);
  // Rows g of the merge list: each group of WPR wavefronts takes a contiguous block of rows
  // (the heads of consecutive tokens of mostly one sequence, whose record it then looks up
  // once); the WPR wavefronts sharing a row see the same g.
  const int nrow_groups = (int)gridDim.x * RPB;
  const int per = (total + nrow_groups - 1) / nrow_groups;
  const int g0 = ((int)blockIdx.x * RPB + wv / WPR) * per;
  const int g1 = min(total, g0 + per);
  SeqHit hit{0, 0};
  int hit_end = 0;  // rows [hit.first, hit_end) belong to sequence hit.s
  SeqInfo si{};
  EntX ex{};
  SeqWork w{};
  for (int g = g0; g < g1; ++g) {
    if (g >= hit_end) {  // wave-uniform
      hit = find_seq(skip, tab, p.pre_g, p.num_ent, g);
      hit_end = wave_uniform(p.pre_g[hit.s + 1]);
      si = seq_record(p, hit.s);
      ex = ent_x(p, hit.s, si.flags);
      w = seq_work(p.is_f32, p.G, p.Hq, p.Hkv, si.q_len, si.L - ex.koff);
    }
    const int local = g - hit.first;
    const int i = local / p.Hq, h = local % p.Hq;
    const int t = si.a + i;
    const int pos = si.L - si.q_len + i;
    // shared partitions, then the row's own ones; later partitions hold no visible key
    const int np = ex.nps + (w.nparts > 0 ? min(w.nparts, (pos - ex.koff) / w.part + 1) : 0);
    const float* base = p.partials + ((int64_t)t * p.Hq + h) * p.maxparts * SF;
    const int c = lane % LPP, qo = lane / LPP;
    float M = kNegInf, l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (np <= WPR * PPI * U) {  // wave-uniform
      // One round trip: every load of the row (the partitions' m and l, lane q holding
      // partition q, and this lane's output columns) is issued before any is used.
      const float* ss = base + (int64_t)(lane < np ? lane : 0) * SF;
      const float ms = ss[D], ls = ss[D + 1];
      f32x4 o[U];
      float mq[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = sub * PPI + qo + u * WPR * PPI;
        const float* sl = base + (int64_t)(q < np ? q : 0) * SF;
        o[u] = *reinterpret_cast<const f32x4*>(sl + 4 * c);
        mq[u] = sl[D];
      }
      M = wave_max(lane < np ? ms : kNegInf);
      // M is finite, so 2^(m - M) is 0 for an empty partition (m = -inf) and for lanes past np
      l = wave_sum(ls * fast_exp2(lane < np ? ms - M : kNegInf));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = sub * PPI + qo + u * WPR * PPI;
        acc += fast_exp2(q < np ? mq[u] - M : kNegInf) * o[u];  // empty partition: weight 0, O_p = 0
      }
    } else {
      // M and l over all partitions; lanes past np read partition 0 and drop it
      for (int q0 = 0; q0 < np; q0 += 64) {
        const int q = q0 + lane;
        const float mq = base[(int64_t)(q < np ? q : 0) * SF + D];
        M = fmaxf(M, q < np ? mq : kNegInf);
      }
      M = wave_max(M);
      float lsum = 0.f;
      for (int q0 = 0; q0 < np; q0 += 64) {
        const int q = q0 + lane;
        const float* sl = base + (int64_t)(q < np ? q : 0) * SF;
        // M is finite, so 2^(m - M) is 0 for an empty partition (m = -inf) and for lanes past np
        const float mq = sl[D], lq = sl[D + 1];
        lsum += lq * fast_exp2(q < np ? mq - M : kNegInf);
      }
      l = wave_sum(lsum);
      // this lane: columns 4c .. 4c + 3 of partitions qo + sub * PPI + k * WPR * PPI
      for (int q0 = sub * PPI; q0 < np; q0 += WPR * PPI * U) {
        f32x4 o[U];
        float mq[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = q0 + qo + u * WPR * PPI;
          const float* sl = base + (int64_t)(q < np ? q : 0) * SF;
          o[u] = *reinterpret_cast<const f32x4*>(sl + 4 * c);
          mq[u] = sl[D];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = q0 + qo + u * WPR * PPI;
          const float wq = fast_exp2(q < np ? mq[u] - M : kNegInf);  // empty partition: weight 0, O_p = 0
          acc += wq * o[u];
        }
      }
    }
#pragma unroll
    for (int off = LPP; off < 64; off <<= 1) {
      acc[0] += shfl_xor_f(acc[0], off);
      acc[1] += shfl_xor_f(acc[1], off);
      acc[2] += shfl_xor_f(acc[2], off);
      acc[3] += shfl_xor_f(acc[3], off);
    }
    if constexpr (WPR > 1) {
      red[wv][lane] = acc;
      __syncthreads();
      acc = red[wv - sub][lane];
#pragma unroll
      for (int k = 1; k < WPR; ++k) acc += red[wv - sub + k][lane];
      __syncthreads();  // red is rewritten for the next row
    }
    // lanes holding the same columns store the same values
    T* orow = (T*)p.out + ((int64_t)t * p.Hq + h) * D + 4 * c;
#pragma unroll
    for (int k = 0; k < 4; ++k) orow[k] = Elem<T>::from_f32(acc[k] / l);
  }
}

// ---------------------------------------------------------------- host side
struct WsLayout {
  size_t ctrl, pre_v, pre_m, pre_t, pre_g, pre_a, pre_b, perm_b, seq_aux, seqinfo, seqx, partials, dec_ctr, total;
  int maxparts;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of a batch of S sequences and NG shared-prefix groups (entries S + NG).
WsLayout ws_layout(int S, int NG, int T, int Hq, int Hkv, int D, int max_ctx, bool is_f32) {
  WsLayout l;
  const int G = Hq / Hkv;
  // group entries split their shared keys in decode-size partitions
  const int part = NG > 0 ? std::min(min_part(is_f32, G), kPartMfmaDecode) : min_part(is_f32, G);
  const int E = S + NG;
  // a member of a group adds at most one partition: its shared and own keys are split separately
  l.maxparts = max(1, (max_ctx + part - 1) / part) + (NG > 0 ? 1 : 0);
  l.ctrl = 0;
  l.pre_v = 512;  // ctrl words 0..63, then the VALU ticket counter on a line of its own
  l.pre_m = l.pre_v + align256((size_t)(E + 1) * 4);
  l.pre_t = l.pre_m + align256((size_t)(E + 1) * 4);
  l.pre_g = l.pre_t + align256((size_t)(E + 1) * 4);
  l.pre_a = l.pre_g + align256((size_t)(E + 1) * 4);
  l.pre_b = l.pre_a + align256((size_t)(E + 1) * 4);
  l.perm_b = l.pre_b + align256((size_t)(S + 1) * 4);
  l.seq_aux = l.perm_b + align256((size_t)S * 4);
  l.seqinfo = l.seq_aux + align256((size_t)S * 8);
  l.seqx = l.seqinfo + align256((size_t)E * 16);
  l.partials = l.seqx + (NG > 0 ? align256((size_t)E * 16) : 0);
  const size_t part_bytes = l.maxparts > 1 ? (size_t)T * Hq * l.maxparts * slot_floats(D) * 4 : 0;
  l.dec_ctr = l.partials + align256(part_bytes);
  l.total = l.dec_ctr + align256((size_t)S * Hkv * 8);
  return l;
}

// Optional events recorded around each stage of pa_forward (see pa_set_stage_events).
thread_local void* const* g_stage_events = nullptr;
thread_local int32_t g_num_stage_events = 0;

inline void mark(int stage, int edge, hipStream_t stream) {
  const int k = 2 * stage + edge;
  if (g_stage_events && k < g_num_stage_events && g_stage_events[k])
    (void)hipEventRecord((hipEvent_t)g_stage_events[k], stream);
}

// Tag of each pa_forward call (the one-pass decode's completion counters).
std::atomic<uint32_t> g_call_tag{1};

template <int D>
void launch_gqa_decode(const AttnParams& p, int grid, hipStream_t stream) {
  mark(0, 0, stream);
  mark(0, 1, stream);
  mark(1, 0, stream);
  mark(1, 1, stream);
  mark(2, 0, stream);
  hipLaunchKernelGGL((gqa_decode_kernel<D>), dim3(grid), dim3(64 * kDecWaves), 0, stream, p);
  mark(2, 1, stream);
  mark(3, 0, stream);
  mark(3, 1, stream);
  mark(4, 0, stream);
  mark(4, 1, stream);
}

// Workgroups of the VALU worker (one wavefront each) that are resident on the current
// device at once, from the occupancy API (cached per device).
template <typename T, int D>
int valu_resident_groups() {
  constexpr int kDevices = 64;
  static std::atomic<int> cached[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < kDevices) {
    const int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int cus = 0, per = 0, n = 4 * kMaxWorkerGroups;
  if (dev >= 0 && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, valu_attn_kernel<T, D>, 64, 0) == hipSuccess && cus > 0 &&
      per > 0)
    n = cus * per;
  if (dev >= 0 && dev < kDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <typename T, int D>
void launch_attention(const AttnParams& p, bool may_valu, bool may_mfma, bool may_tile, int64_t bound_v,
                      int grid_m, int grid_t, hipStream_t stream) {
  // a strided batch (sequences sharing pages) uses all of the VALU grid, a ticket batch its
  // resident part; the grid is a multiple of 32 (the strided order permutes blocks of 32)
  AttnParams pv = p;
  int64_t grid_v = 32;
  if (may_valu) {
    const int64_t res = valu_resident_groups<T, D>();
    grid_v = std::min<int64_t>(std::max<int64_t>(32, kValuGridPerResident * res / 32 * 32),
                               std::max<int64_t>(32, (bound_v + 31) / 32 * 32));
    pv.valu_resident = (int32_t)std::min<int64_t>(res, grid_v);
    pv.len_order_ok = bound_v < (int64_t)kLenOrderItems * pv.valu_resident ? 1 : 0;
  }
  mark(0, 0, stream);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, pv);
  mark(0, 1, stream);
  mark(1, 0, stream);
  if (may_valu) hipLaunchKernelGGL((valu_attn_kernel<T, D>), dim3((unsigned)grid_v), dim3(64), 0, stream, pv);
  mark(1, 1, stream);
  mark(2, 0, stream);
  if constexpr (sizeof(T) == 2)
    if (may_mfma) hipLaunchKernelGGL((mfma_attn_kernel<D>), dim3(grid_m), dim3(256), 0, stream, p);
  mark(2, 1, stream);
  mark(3, 0, stream);
  if constexpr (sizeof(T) == 2)
    if (may_tile)
      hipLaunchKernelGGL((tile_attn_kernel<D>), dim3(grid_t), dim3(64 * kTileWaves), 0, stream, p);
  mark(3, 1, stream);
  mark(4, 0, stream);
  if (p.maxparts > 1) {
    // many partitions per row (long contexts): four wavefronts share a row
    const int64_t rows = (int64_t)p.T * p.Hq;  // bound on the rows to merge
    if (p.maxparts >= kMergeSplitParts)
      hipLaunchKernelGGL((merge_kernel<T, D, 4>), dim3((unsigned)std::min<int64_t>(kMaxWorkerGroups, rows)),
                         dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<T, D, 1>), dim3((unsigned)std::min<int64_t>(kMaxWorkerGroups, (rows + 3) / 4)),
                         dim3(256), 0, stream, p);
  }
  mark(4, 1, stream);
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" size_t pa_forward_workspace_bytes(int32_t num_seqs, int32_t total_q_tokens,
                                             int32_t max_q_len, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, pa_dtype dtype) {
  (void)max_q_len;
  if (num_seqs < 0 || total_q_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_context_len < 0 || num_q_heads % num_kv_heads)
    return 0;
  return ws_layout(num_seqs, 0, total_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len,
                   dtype == PA_F32)
      .total;
}

extern "C" size_t pa_forward_shared_workspace_bytes(int32_t num_seqs, int32_t num_groups, int32_t total_q_tokens,
                                                    int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_dim, int32_t max_context_len, pa_dtype dtype) {
  (void)max_q_len;
  if (num_seqs < 0 || num_groups < 0 || total_q_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_context_len < 0 || num_q_heads % num_kv_heads)
    return 0;
  return ws_layout(num_seqs, num_groups, total_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len,
                   dtype == PA_F32)
      .total;
}

namespace {

pa_status forward_impl(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* query_start_loc, const int32_t* groups, int32_t num_groups,
                       int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                       int32_t* dev_status, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (block_size != kBlock)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, head_dim);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PA_ERR_INVALID, "%s: %d query heads are not a multiple of %d KV heads", fn,
                num_q_heads, num_kv_heads);
  if (num_seqs < 0 || total_q_tokens < 0 || max_q_len < 0 || max_context_len < 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID, "%s: negative size or empty pool", fn);
  if (max_q_len > max_context_len || max_q_len > total_q_tokens)
    return fail(PA_ERR_INVALID, "%s: max_q_len %d exceeds max_context_len %d or total_q_tokens %d",
                fn, max_q_len, max_context_len, total_q_tokens);
  if ((int64_t)max_blocks_per_seq * kBlock < max_context_len || max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq %d cannot hold %d tokens", fn,
                max_blocks_per_seq, max_context_len);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "%s: scale is not finite", fn);
  if ((int64_t)total_q_tokens * num_q_heads > INT32_MAX / 2)
    return fail(PA_ERR_INVALID, "%s: batch too large", fn);
  if (num_seqs == 0 || total_q_tokens == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc ||
      !workspace)
    return fail(PA_ERR_INVALID, "%s: NULL device pointer", fn);
  if ((uintptr_t)workspace % 256) return fail(PA_ERR_INVALID, "%s: workspace not 256-byte aligned", fn);
  const bool is_f32 = dtype == PA_F32;
  if (num_groups < 0 || (num_groups > 0 && !groups)) return fail(PA_ERR_INVALID, "%s: bad group list", fn);
  if (num_groups > 0 && (is_f32 || 2 * (num_q_heads / num_kv_heads) > kTileRows))
    return fail(PA_ERR_UNSUPPORTED, "%s: shared prefixes need bfloat16 and at most %d query heads per KV head", fn,
                kTileRows / 2);
  if (num_groups > num_seqs) return fail(PA_ERR_INVALID, "%s: %d groups for %d sequences", fn, num_groups, num_seqs);
  const WsLayout wl = ws_layout(num_seqs, num_groups, total_q_tokens, num_q_heads, num_kv_heads, head_dim,
                                max_context_len, is_f32);
  if (workspace_bytes < wl.total)
    return fail(PA_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, wl.total);

  AttnParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.qsl = query_start_loc;
  p.mbps = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.T = total_q_tokens;
  p.max_q_len = max_q_len;
  p.max_ctx = max_context_len;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.G = num_q_heads / num_kv_heads;
  p.num_blocks = num_blocks;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.is_f32 = is_f32;
  char* ws = (char*)workspace;
  p.ctrl = (int32_t*)(ws + wl.ctrl);
  p.pre_v = (int32_t*)(ws + wl.pre_v);
  p.pre_m = (int32_t*)(ws + wl.pre_m);
  p.pre_t = (int32_t*)(ws + wl.pre_t);
  p.pre_g = (int32_t*)(ws + wl.pre_g);
  p.pre_a = (int32_t*)(ws + wl.pre_a);
  p.pre_b = (int32_t*)(ws + wl.pre_b);
  p.perm_b = (int32_t*)(ws + wl.perm_b);
  p.seq_aux = (int32_t*)(ws + wl.seq_aux);
  p.seqinfo = (i32x4*)(ws + wl.seqinfo);
  p.partials = (float*)(ws + wl.partials);
  p.maxparts = wl.maxparts;
  p.dev_status = dev_status;
  p.num_ent = num_seqs + num_groups;
  p.groups = groups;
  p.num_groups = num_groups;
  p.seqx = num_groups > 0 ? (i32x4*)(ws + wl.seqx) : nullptr;
  p.dec_ctr = (unsigned long long*)(ws + wl.dec_ctr);
  p.call_tag = g_call_tag.fetch_add(1, std::memory_order_relaxed);
  hipStream_t s = (hipStream_t)stream;

  // Single-position GQA decode batches run in one dispatch (no planner, no merge kernel).
  if (!is_f32 && num_groups == 0 && max_q_len == 1 && p.G >= 2 && p.G <= kTileRows) {
    const int64_t chunks = std::max(1, dec_chunks(max_context_len));
    const int64_t grid = (int64_t)num_seqs * num_kv_heads * chunks;
    if (grid > INT32_MAX) return fail(PA_ERR_INVALID, "%s: batch too large", fn);
    (void)hipGetLastError();
    if (head_dim == 64) launch_gqa_decode<64>(p, (int)grid, s);
    else launch_gqa_decode<128>(p, (int)grid, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
  }

  // Which worker classes can receive items (decided from host-known bounds only).
  const bool may_valu = is_f32 || p.G == 1;
  const bool may_mfma = !is_f32 && p.G <= kTileRows && (p.G > 1 || max_q_len > 1 || num_groups > 0);
  const bool may_tile = !is_f32 && (int64_t)max_q_len * p.G > kTileRows;
  const int64_t bound_v = (int64_t)total_q_tokens * num_q_heads * wl.maxparts;
  const int64_t bound_m = (int64_t)(num_seqs + num_groups) * num_kv_heads * wl.maxparts;
  const int64_t bound_t =
      ((int64_t)total_q_tokens * p.G / kBigRows + num_seqs) * num_kv_heads * wl.maxparts;
  const int grid_m = (int)std::min<int64_t>(kMaxWorkerGroups, (bound_m + 3) / 4);
  const int grid_t = (int)std::min<int64_t>(kMaxTileGroups, bound_t);

  (void)hipGetLastError();
  if (is_f32) {
    if (head_dim == 64) launch_attention<float, 64>(p, may_valu, false, false, bound_v, grid_m, grid_t, s);
    else launch_attention<float, 128>(p, may_valu, false, false, bound_v, grid_m, grid_t, s);
  } else {
    if (head_dim == 64) launch_attention<bf16_t, 64>(p, may_valu, may_mfma, may_tile, bound_v, grid_m, grid_t, s);
    else launch_attention<bf16_t, 128>(p, may_valu, may_mfma, may_tile, bound_v, grid_m, grid_t, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" pa_status pa_forward(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                float scale, pa_dtype dtype, void* workspace,
                                size_t workspace_bytes, int32_t* dev_status, void* stream) {
  return forward_impl("pa_forward", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                      query_start_loc, nullptr, 0, num_seqs, total_q_tokens, max_q_len, max_context_len,
                      num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype, workspace,
                      workspace_bytes, dev_status, stream);
}

extern "C" pa_status pa_forward_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, const int32_t* query_start_loc,
                                       const int32_t* groups, int32_t num_groups, int32_t num_seqs,
                                       int32_t total_q_tokens, int32_t max_q_len, int32_t max_context_len,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, float scale, pa_dtype dtype,
                                       void* workspace, size_t workspace_bytes, int32_t* dev_status,
                                       void* stream) {
  return forward_impl("pa_forward_shared", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                      context_lens, query_start_loc, groups, num_groups, num_seqs, total_q_tokens, max_q_len,
                      max_context_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                      workspace, workspace_bytes, dev_status, stream);
}

extern "C" pa_status pa_set_stage_events(void* const* events, int32_t num_events) {
  if (num_events < 0 || (num_events > 0 && !events))
    return fail(PA_ERR_INVALID, "pa_set_stage_events: bad event list");
  g_stage_events = num_events ? events : nullptr;
  g_num_stage_events = num_events;
  return ok();
}

// ---------------------------------------------------------------- without allocation
// Workspace of pa_forward_noalloc: one array per GPU, in the code object's
// device data, held from the library's load until the process ends.  Host code
// never passes the array's own name to a kernel (on the host it is only a
// stand-in); it takes the device address from hipGetSymbolAddress, once per
// device with that device current, and passes that.
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pa_status scratch_of_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}
}  // namespace

extern "C" size_t pa_forward_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

extern "C" pa_status pa_forward_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, const int32_t* query_start_loc,
                                        int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                        int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                        pa_dtype dtype, int32_t* dev_status, void* stream) {
  const char* fn = "pa_forward_noalloc";
  const size_t need = pa_forward_workspace_bytes(num_seqs, total_q_tokens, max_q_len, num_q_heads, num_kv_heads,
                                                 head_dim, max_context_len, dtype);
  if (need > kScratchBytes)
    return fail(PA_ERR_INVALID, "%s: this batch needs %zu bytes of workspace, the static workspace holds %zu", fn,
                need, kScratchBytes);
  void* ws = nullptr;
  if (num_seqs > 0 && total_q_tokens > 0) {
    const pa_status st = scratch_of_current_device(fn, &ws);
    if (st != PA_OK) return st;
  }
  return forward_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, query_start_loc,
                      nullptr, 0, num_seqs, total_q_tokens, max_q_len, max_context_len, num_q_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, scale, dtype, ws, kScratchBytes, dev_status, stream);
}
