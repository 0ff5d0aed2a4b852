// C ABI of libpa: argument checks, the split-schedule plan, workspace
// layout and kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_launch.h"

namespace {

constexpr int kAbiVersion = 3;
// Upper bound on 64-lane workgroups per compute unit the schedule aims for;
// the kernel's register budget may allow fewer.  Measured on MI355X: four
// per CU streams as fast as eight or more while giving each range twice the
// blocks, so fewer sequences are split and fewer partials are merged.
constexpr int kWavesPerCu = 4;
// Fewest KV blocks a range should hold before more ranges stop paying off.
constexpr int kMinBlocksPerRange = 8;
constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 0;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || n <= 0)
      return 0;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Scratch of pa_decode_append_noalloc (block prefix sums and split-context
// partials, the same contents as the workspace of pa_decode_append), for
// callers that cannot allocate.  Every device the library runs on holds
// one copy from the time the library's code is loaded on it until the
// process ends.  Host code never uses the array's name as an address: the
// device address of each device's copy is resolved once, with that device
// current, by scratch_on_device().
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, or nullptr when it
// cannot be resolved.
void* scratch_on_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t dtype_bytes(pa_dtype t) {
  switch (t) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_FP8_E4M3FN: return 1;
  }
  return 0;
}

bool head_size_ok(int d) { return d == 64 || d == 128 || d == 256; }

int check_desc(const pa_decode_desc* d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_seqs < 0 || d->num_seqs > 65536) return PA_ERR_SHAPE;
  if (d->num_kv_heads < 1 || d->num_q_heads < d->num_kv_heads ||
      d->num_q_heads % d->num_kv_heads)
    return PA_ERR_SHAPE;
  if (!head_size_ok(d->head_size) || d->block_size != pa::kBlock)
    return PA_ERR_SHAPE;
  if (d->num_blocks < 1 ||
      (int64_t)d->num_blocks * pa::kBlock > INT32_MAX)
    return PA_ERR_SHAPE;
  if (d->max_blocks_per_seq < 1 || d->max_seq_len < 0) return PA_ERR_SHAPE;
  // per-head block counts and their prefix sums stay in int32
  if ((int64_t)d->num_seqs * d->max_blocks_per_seq > INT32_MAX)
    return PA_ERR_SHAPE;
  if (d->num_waves < 0 || d->total_blocks_hint < 0) return PA_ERR_SHAPE;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->q_dtype == PA_F32 && d->kv_dtype == PA_F32) {
    if (G > 8) return PA_ERR_SHAPE;
  } else if (d->q_dtype == PA_BF16 &&
             (d->kv_dtype == PA_BF16 || d->kv_dtype == PA_FP8_E4M3FN)) {
    if (G > 16) return PA_ERR_SHAPE;
  } else {
    return PA_ERR_DTYPE;
  }
  if (d->kv_dtype == PA_FP8_E4M3FN &&
      !(d->k_scale > 0.f && d->v_scale > 0.f && isfinite(d->k_scale) &&
        isfinite(d->v_scale)))
    return PA_ERR_SHAPE;
  return PA_OK;
}

struct Plan {
  int Wh;  // ranges per KV head
  int W;   // workgroups of the main pass
  size_t off_ml, off_o, off_dml, off_do, bytes;
  // cascade decode: suffix tables and lengths, shared-prefix partials
  size_t off_st, off_sl, off_sml, off_so;
  int splits;  // key ranges per group of the shared-prefix pass
};

// Ranges per KV head: enough resident workgroups to fill every CU, but no
// range shorter than kMinBlocksPerRange blocks when the total is known or
// bounded.
bool make_plan(const pa_decode_desc* d, bool fused, Plan* p,
               bool cascade = false) {
  const int hkv = d->num_kv_heads;
  const int G = d->num_q_heads / hkv;
  int64_t wh;
  if (d->num_waves > 0) {
    wh = d->num_waves / hkv;
  } else {
    const int cus = cu_count();
    if (cus <= 0) return false;
    int per_cu = d->kv_dtype == PA_F32
                     ? pa::occupancy_decode_valu(d->head_size)
                     : pa::occupancy_decode_mfma(
                           d->kv_dtype == PA_FP8_E4M3FN, d->head_size);
    if (per_cu <= 0) return false;
    // Twice as many ranges when a pair of blocks carries 4 KiB or less (fp8
    // at D = 64): such waves hold too few bytes in flight to stream the pool
    // at four per compute unit (measured: 26.0 against 28.7 us on the
    // Llama-shaped batch at D = 64; at D = 128 fp8 and at D = 64 bf16, eight
    // per compute unit are 1.5% and 2% slower).
    const int64_t pair_bytes = 64 * (int64_t)d->head_size *
                               (int64_t)dtype_bytes(d->kv_dtype);
    const int per_cu_cap = d->kv_dtype != PA_F32 && pair_bytes <= 4096
                               ? 2 * kWavesPerCu
                               : kWavesPerCu;
    if (per_cu > per_cu_cap) per_cu = per_cu_cap;
    wh = (int64_t)cus * per_cu / hkv;
    int64_t units = d->total_blocks_hint;
    if (units <= 0) {
      int64_t per = (d->max_seq_len + pa::kBlock - 1) / pa::kBlock;
      if (per > d->max_blocks_per_seq) per = d->max_blocks_per_seq;
      units = (int64_t)d->num_seqs * per;
    }
    int64_t cap = (units + kMinBlocksPerRange - 1) / kMinBlocksPerRange;
    if (wh > cap) wh = cap;
  }
  if (wh < 1) wh = 1;
  if (wh * hkv > INT32_MAX / 2) wh = INT32_MAX / 2 / hkv;
  p->Wh = (int)wh;
  p->W = (int)(wh * hkv);
  const size_t rows = (size_t)p->W * 2 * G;
  const size_t prefix = round_up(((size_t)d->num_seqs + 1) * sizeof(int32_t));
  p->off_ml = prefix;
  p->off_o = p->off_ml + round_up(rows * 2 * sizeof(float));
  p->bytes = p->off_o + round_up(rows * d->head_size * sizeof(float));
  p->off_dml = p->off_do = 0;
  if (fused) {  // direct partials, one per (sequence, query head)
    const size_t hrows = (size_t)d->num_seqs * d->num_q_heads;
    p->off_dml = p->bytes;
    p->off_do = p->off_dml + round_up(hrows * 2 * sizeof(float));
    p->bytes = p->off_do + round_up(hrows * d->head_size * sizeof(float));
  }
  p->off_st = p->off_sl = p->off_sml = p->off_so = 0;
  p->splits = 1;
  if (cascade) {
    // Key ranges per shared prefix: about one workgroup per CU when one
    // group covers the batch (measured on MI355X with a 128-sequence batch
    // sharing 2048 tokens: two per CU or a half per CU is slower, the first
    // by the extra partials the merge reads), at least two 64-key steps per
    // range of the longest possible prefix, at most kMaxSharedSplits.
    const int cus = cu_count();
    if (cus <= 0) return false;
    const int64_t tiles =
        ((int64_t)d->num_seqs * G + pa::kPrefillWaves * 32 - 1) /
            (pa::kPrefillWaves * 32) + 1;
    int64_t ns = ((int64_t)cus + tiles * hkv - 1) / (tiles * hkv);
    const int64_t steps_cap = ((d->max_seq_len + 63) / 64 + 1) / 2;
    if (ns > steps_cap) ns = steps_cap;
    if (ns > pa::kMaxSharedSplits) ns = pa::kMaxSharedSplits;
    if (ns < 1) ns = 1;
    p->splits = (int)ns;
    const size_t hrows = (size_t)d->num_seqs * d->num_q_heads * ns;
    p->off_st = p->bytes;
    p->off_sl = p->off_st + round_up((size_t)d->num_seqs *
                                     d->max_blocks_per_seq * sizeof(int32_t));
    p->off_sml = p->off_sl + round_up((size_t)d->num_seqs * sizeof(int32_t));
    p->off_so = p->off_sml + round_up(hrows * 2 * sizeof(float));
    p->bytes = p->off_so + round_up(hrows * d->head_size * sizeof(float));
  }
  return true;
}

// Groups of a cascade decode call (device arrays).
struct SharedPrefix {
  const int32_t* group_start;          // [num_groups + 1]
  const int32_t* group_prefix_blocks;  // [num_groups]
  int num_groups;
};

// All decode entry points; k_new == nullptr selects the plain decode, sp
// the cascade form of the fused step.
int run_decode(const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, const int32_t* seq_lens,
               float scale, void* out, const void* k_new, const void* v_new,
               const int32_t* slots, void* k_pool_w, void* v_pool_w,
               const pa_decode_desc* desc, void* workspace,
               size_t workspace_bytes, void* stream,
               const SharedPrefix* sp = nullptr) {
  int st = check_desc(desc);
  if (st != PA_OK) return st;
  const bool fused = k_new != nullptr;
  if (sp) {
    if (desc->q_dtype != PA_BF16 ||
        (desc->kv_dtype != PA_BF16 && desc->kv_dtype != PA_FP8_E4M3FN))
      return PA_ERR_DTYPE;
    if ((desc->head_size != 64 && desc->head_size != 128) ||
        sp->num_groups < 0 || sp->num_groups > desc->num_seqs)
      return PA_ERR_SHAPE;
    if (!(scale > 0.f)) return PA_ERR_SHAPE;
    const int G = desc->num_q_heads / desc->num_kv_heads;
    if (pa::prefill_grid(desc->head_size, desc->num_seqs, G, sp->num_groups,
                         desc->num_kv_heads) * pa::kMaxSharedSplits +
            desc->num_seqs > INT32_MAX)
      return PA_ERR_SHAPE;
  }
  if (desc->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out)
    return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(out) || ((uintptr_t)block_tables & 3u) ||
      ((uintptr_t)seq_lens & 3u))
    return PA_ERR_ALIGN;
  if (fused && (!aligned16(k_new) || !aligned16(v_new) ||
                ((uintptr_t)slots & 3u)))
    return PA_ERR_ALIGN;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  if (sp && sp->num_groups > 0) {
    if (!sp->group_start || !sp->group_prefix_blocks) return PA_ERR_NULL;
    if (((uintptr_t)sp->group_start & 3u) ||
        ((uintptr_t)sp->group_prefix_blocks & 3u))
      return PA_ERR_ALIGN;
  }
  Plan p;
  if (!make_plan(desc, fused, &p, sp != nullptr)) return PA_ERR_DEVICE;
  if (!workspace || workspace_bytes < p.bytes) return PA_ERR_WORKSPACE;
  if ((uintptr_t)workspace % kAlign) return PA_ERR_ALIGN;

  char* ws = static_cast<char*>(workspace);
  pa::DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.prefix = reinterpret_cast<int32_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + p.off_ml);
  a.part_o = reinterpret_cast<float*>(ws + p.off_o);
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slots;
  a.k_pool_w = k_pool_w;
  a.v_pool_w = v_pool_w;
  a.direct_ml = fused ? reinterpret_cast<float*>(ws + p.off_dml) : nullptr;
  a.direct_o = fused ? reinterpret_cast<float*>(ws + p.off_do) : nullptr;
  const float k_scale = desc->kv_dtype == PA_FP8_E4M3FN ? desc->k_scale : 1.f;
  a.s.c_log2 = (float)((double)scale * 1.4426950408889634 * (double)k_scale);
  a.s.v_scale = desc->kv_dtype == PA_FP8_E4M3FN ? desc->v_scale : 1.f;
  a.s.Hq = desc->num_q_heads;
  a.s.NB = desc->num_blocks;
  a.s.B = desc->num_seqs;
  a.s.max_blocks = desc->max_blocks_per_seq;
  a.s.Hkv = desc->num_kv_heads;
  a.s.G = desc->num_q_heads / desc->num_kv_heads;
  a.s.Wh = p.Wh;
  a.s.len_bias = fused ? 1 : 0;
  a.shared_ml = nullptr;
  a.shared_o = nullptr;
  a.shared_splits = 0;
  a.full_lens = nullptr;
  a.merge_pairs = false;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t* ev = reinterpret_cast<hipEvent_t*>(
      const_cast<void**>(desc->profile_events));
  // the cascade step's events bracket all of its launches
  const bool cascade = sp && sp->num_groups > 0;
  if (cascade && ev[0] && hipEventRecord(ev[0], s) != hipSuccess)
    return PA_ERR_LAUNCH;
  if (cascade) {
    // one launch reads the shared prefixes once per group and writes the
    // suffix view of every sequence; the main and merge passes below run
    // on the suffixes
    int32_t* st_tab = reinterpret_cast<int32_t*>(ws + p.off_st);
    int32_t* st_len = reinterpret_cast<int32_t*>(ws + p.off_sl);
    float* sml = reinterpret_cast<float*>(ws + p.off_sml);
    float* so = reinterpret_cast<float*>(ws + p.off_so);
    pa::PrefillArgs pf;
    pf.q = q;
    pf.k_pool = k_pool;
    pf.v_pool = v_pool;
    pf.block_tables = block_tables;
    pf.seq_lens = sp->group_prefix_blocks;
    pf.q_start = sp->group_start;
    pf.out = nullptr;
    pf.member_lens = seq_lens;
    pf.part_ml = sml;
    pf.part_o = so;
    pf.suffix_tables = st_tab;
    pf.suffix_lens = st_len;
    pf.s.B = sp->num_groups;
    pf.s.Hq = desc->num_q_heads;
    pf.s.Hkv = desc->num_kv_heads;
    pf.s.G = a.s.G;
    pf.s.max_blocks = desc->max_blocks_per_seq;
    pf.s.NB = desc->num_blocks;
    pf.s.T = desc->num_seqs;
    pf.s.c_log2 = a.s.c_log2;
    pf.s.v_scale = a.s.v_scale;
    pf.s.splits = p.splits;
    const hipError_t e = pa::launch_shared_prefix(
        desc->head_size, desc->kv_dtype == PA_FP8_E4M3FN, pf, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;

    a.block_tables = st_tab;
    a.seq_lens = st_len;
    a.full_lens = seq_lens;
    a.shared_ml = sml;
    a.shared_o = so;
    a.shared_splits = p.splits;
  }
  // outside the cascade step the events ride on the main kernel's own
  // dispatch: they time the kernel alone, with no packets of their own
  a.ev_start = cascade ? nullptr : ev[0];
  a.ev_stop = cascade ? nullptr : ev[1];
  hipError_t e;
  if (desc->kv_dtype == PA_F32)
    e = pa::launch_decode_valu(desc->head_size, a, p.W, s);
  else
    e = pa::launch_decode_mfma(desc->kv_dtype == PA_FP8_E4M3FN,
                               desc->head_size, a, p.W, s);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  a.ev_start = a.ev_stop = nullptr;
  if (fused) {
    // One query head per merge wave while the whole grid fits on the GPU
    // at once (more loads in flight); two per wave beyond that, so a large
    // batch still takes one round of waves.
    const int kb = (int)dtype_bytes(desc->kv_dtype);
    const int64_t resident =
        (int64_t)pa::occupancy_decode_merge_append(kb, desc->head_size) *
        cu_count();
    a.merge_pairs = !a.shared_ml && resident > 0 &&
                    (int64_t)desc->num_seqs * desc->num_q_heads > resident;
    e = pa::launch_decode_merge_append(kb, desc->head_size, a, s);
  } else {
    const bool bf16 = desc->q_dtype == PA_BF16;
    const int64_t resident =
        (int64_t)pa::occupancy_decode_merge(bf16, desc->head_size) *
        cu_count();
    a.merge_pairs = resident > 0 &&
                    (int64_t)desc->num_seqs * desc->num_q_heads > resident;
    e = pa::launch_decode_merge(bf16, desc->head_size, a, s);
  }
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  if (cascade && ev[1] && hipEventRecord(ev[1], s) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return kAbiVersion; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_DTYPE: return "unsupported dtype combination";
    case PA_ERR_SHAPE: return "unsupported or inconsistent size";
    case PA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_DEVICE: return "no usable HIP device";
    case PA_ERR_SCRATCH:
      return "call needs more than the library's static scratch buffer";
  }
  return "unknown status";
}

size_t pa_decode_workspace_size(const pa_decode_desc* desc) {
  if (check_desc(desc) != PA_OK) return 0;
  if (desc->num_seqs == 0) return 0;
  Plan p;
  if (!make_plan(desc, false, &p)) return 0;
  return p.bytes;
}

size_t pa_decode_append_workspace_size(const pa_decode_desc* desc) {
  if (check_desc(desc) != PA_OK) return 0;
  if (desc->num_seqs == 0) return 0;
  Plan p;
  if (!make_plan(desc, true, &p)) return 0;
  return p.bytes;
}

int pa_decode(const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* seq_lens,
              float scale, void* out, const pa_decode_desc* desc,
              void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                    nullptr, nullptr, nullptr, nullptr, nullptr, desc,
                    workspace, workspace_bytes, stream);
}

int pa_decode_append(const void* q, void* k_pool, void* v_pool,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     float scale, void* out, const void* k_new,
                     const void* v_new, const int32_t* slot_mapping,
                     const pa_decode_desc* desc, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!desc) return PA_ERR_NULL;
  if (desc->num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return PA_ERR_NULL;
  if (desc->num_seqs == 0) return check_desc(desc);
  return run_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                    k_new, v_new, slot_mapping, k_pool, v_pool, desc,
                    workspace, workspace_bytes, stream);
}

int pa_decode_append_noalloc(const void* q, void* k_pool, void* v_pool,
                             const int32_t* block_tables,
                             const int32_t* seq_lens, float scale, void* out,
                             const void* k_new, const void* v_new,
                             const int32_t* slot_mapping,
                             const pa_decode_desc* desc, void* stream) {
  if (!desc) return PA_ERR_NULL;
  if (desc->num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return PA_ERR_NULL;
  const int st = check_desc(desc);
  if (st != PA_OK || desc->num_seqs == 0) return st;
  Plan p;
  if (!make_plan(desc, true, &p)) return PA_ERR_DEVICE;
  if (p.bytes > kScratchBytes) return PA_ERR_SCRATCH;
  void* ws = scratch_on_device();
  if (!ws) return PA_ERR_DEVICE;
  return run_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                    k_new, v_new, slot_mapping, k_pool, v_pool, desc, ws,
                    kScratchBytes, stream);
}

size_t pa_decode_append_shared_workspace_size(const pa_decode_desc* desc) {
  if (check_desc(desc) != PA_OK) return 0;
  if (desc->num_seqs == 0) return 0;
  Plan p;
  if (!make_plan(desc, true, &p, true)) return 0;
  return p.bytes;
}

int pa_decode_append_shared(const void* q, void* k_pool, void* v_pool,
                            const int32_t* block_tables,
                            const int32_t* seq_lens, float scale, void* out,
                            const void* k_new, const void* v_new,
                            const int32_t* slot_mapping,
                            const int32_t* group_start,
                            const int32_t* group_prefix_blocks,
                            int32_t num_groups, const pa_decode_desc* desc,
                            void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!desc) return PA_ERR_NULL;
  if (desc->num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return PA_ERR_NULL;
  if (desc->num_seqs == 0) return check_desc(desc);
  SharedPrefix sp{group_start, group_prefix_blocks, num_groups};
  return run_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out,
                    k_new, v_new, slot_mapping, k_pool, v_pool, desc,
                    workspace, workspace_bytes, stream, &sp);
}

int pa_kv_append(const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, void* k_pool, void* v_pool,
                 const pa_append_desc* desc, void* stream) {
  if (!desc) return PA_ERR_NULL;
  if (desc->num_tokens < 0 || desc->num_kv_heads < 1 ||
      !head_size_ok(desc->head_size) || desc->block_size != pa::kBlock ||
      desc->num_blocks < 1 ||
      (int64_t)desc->num_blocks * pa::kBlock > INT32_MAX)
    return PA_ERR_SHAPE;
  const size_t eb = dtype_bytes(desc->kv_dtype);
  if (eb == 0) return PA_ERR_DTYPE;
  if ((int64_t)desc->num_kv_heads * desc->head_size > INT32_MAX / 16 ||
      pa::append_workgroups(desc->num_tokens, desc->num_kv_heads) >
          INT32_MAX)
    return PA_ERR_SHAPE;
  if (desc->num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool)
    return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) ||
      !aligned16(v_pool) || ((uintptr_t)slot_mapping & 3u))
    return PA_ERR_ALIGN;
  hipError_t e = pa::launch_kv_append(
      (int)eb, k_new, v_new, slot_mapping, k_pool, v_pool, desc->num_tokens,
      desc->num_kv_heads, desc->head_size, desc->num_blocks,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_kv_append_quant(const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, void* k_pool,
                       void* v_pool, const pa_append_desc* desc,
                       float k_scale, float v_scale, void* stream) {
  if (!desc) return PA_ERR_NULL;
  if (desc->num_tokens < 0 || desc->num_kv_heads < 1 ||
      !head_size_ok(desc->head_size) || desc->block_size != pa::kBlock ||
      desc->num_blocks < 1 ||
      (int64_t)desc->num_blocks * pa::kBlock > INT32_MAX)
    return PA_ERR_SHAPE;
  if (desc->kv_dtype != PA_FP8_E4M3FN) return PA_ERR_DTYPE;
  if (!(k_scale > 0.f && v_scale > 0.f && isfinite(k_scale) &&
        isfinite(v_scale)))
    return PA_ERR_SHAPE;
  if ((int64_t)desc->num_kv_heads * desc->head_size > INT32_MAX / 16 ||
      pa::append_workgroups(desc->num_tokens, desc->num_kv_heads) >
          INT32_MAX)
    return PA_ERR_SHAPE;
  if (desc->num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool)
    return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) ||
      !aligned16(v_pool) || ((uintptr_t)slot_mapping & 3u))
    return PA_ERR_ALIGN;
  hipError_t e = pa::launch_kv_append_quant(
      k_new, v_new, slot_mapping, k_pool, v_pool, desc->num_tokens,
      desc->num_kv_heads, desc->head_size, desc->num_blocks, k_scale,
      v_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                   const int32_t* dst_blocks, const pa_copy_desc* desc,
                   void* stream) {
  if (!desc) return PA_ERR_NULL;
  if (desc->num_pairs < 0 || desc->num_kv_heads < 1 ||
      !head_size_ok(desc->head_size) || desc->block_size != pa::kBlock ||
      desc->num_blocks < 1)
    return PA_ERR_SHAPE;
  const size_t eb = dtype_bytes(desc->kv_dtype);
  if (eb == 0) return PA_ERR_DTYPE;
  const int64_t block_bytes =
      (int64_t)desc->num_kv_heads * pa::kBlock * desc->head_size * (int64_t)eb;
  if (block_bytes > INT32_MAX / 2) return PA_ERR_SHAPE;
  if ((int64_t)desc->num_pairs *
          pa::copy_workgroups_per_pair((int)block_bytes) >
      INT32_MAX)
    return PA_ERR_SHAPE;
  if (desc->num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_blocks || !dst_blocks) return PA_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)src_blocks & 3u) || ((uintptr_t)dst_blocks & 3u))
    return PA_ERR_ALIGN;
  hipError_t e = pa::launch_copy_blocks(
      k_pool, v_pool, src_blocks, dst_blocks, desc->num_pairs,
      (int)block_bytes, desc->num_blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_prefill(const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, const int32_t* seq_lens,
               const int32_t* q_start, float scale, void* out,
               const pa_prefill_desc* desc, void* stream) {
  if (!desc) return PA_ERR_NULL;
  const pa_prefill_desc* d = desc;
  if (d->num_seqs < 0 || d->num_seqs > 65536 || d->num_query_tokens < 0)
    return PA_ERR_SHAPE;
  if (d->num_kv_heads < 1 || d->num_q_heads < d->num_kv_heads ||
      d->num_q_heads % d->num_kv_heads ||
      d->num_q_heads / d->num_kv_heads > 16)
    return PA_ERR_SHAPE;
  if ((d->head_size != 64 && d->head_size != 128) ||
      d->block_size != pa::kBlock)
    return PA_ERR_SHAPE;
  if (d->num_blocks < 1 || (int64_t)d->num_blocks * pa::kBlock > INT32_MAX ||
      d->max_blocks_per_seq < 1 ||
      (int64_t)d->max_blocks_per_seq * pa::kBlock > INT32_MAX)
    return PA_ERR_SHAPE;
  if (d->q_dtype != PA_BF16 ||
      (d->kv_dtype != PA_BF16 && d->kv_dtype != PA_FP8_E4M3FN))
    return PA_ERR_DTYPE;
  const bool fp8 = d->kv_dtype == PA_FP8_E4M3FN;
  if (fp8 && !(d->k_scale > 0.f && d->v_scale > 0.f && isfinite(d->k_scale) &&
               isfinite(d->v_scale)))
    return PA_ERR_SHAPE;
  const int G = d->num_q_heads / d->num_kv_heads;
  if ((int64_t)d->num_query_tokens * d->num_q_heads > INT32_MAX ||
      pa::prefill_grid(d->head_size, d->num_query_tokens, G, d->num_seqs,
                       d->num_kv_heads) > INT32_MAX)
    return PA_ERR_SHAPE;
  if (!isfinite(scale) || !(scale > 0.f)) return PA_ERR_SHAPE;
  if (d->num_seqs == 0 || d->num_query_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !q_start ||
      !out)
    return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(out) || ((uintptr_t)block_tables & 3u) ||
      ((uintptr_t)seq_lens & 3u) || ((uintptr_t)q_start & 3u))
    return PA_ERR_ALIGN;
  pa::PrefillArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.q_start = q_start;
  a.out = out;
  a.s.B = d->num_seqs;
  a.s.Hq = d->num_q_heads;
  a.s.Hkv = d->num_kv_heads;
  a.s.G = G;
  a.s.max_blocks = d->max_blocks_per_seq;
  a.s.NB = d->num_blocks;
  a.s.T = d->num_query_tokens;
  a.s.c_log2 = (float)((double)scale * 1.4426950408889634 *
                       (fp8 ? (double)d->k_scale : 1.0));
  a.s.v_scale = fp8 ? d->v_scale : 1.f;
  a.s.splits = 1;
  a.s.attn_grid = 0;
  a.member_lens = nullptr;
  a.suffix_tables = nullptr;
  a.suffix_lens = nullptr;
  a.part_ml = nullptr;
  a.part_o = nullptr;
  hipError_t e =
      pa::launch_prefill(d->head_size, fp8, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
