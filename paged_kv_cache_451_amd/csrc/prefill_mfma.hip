// Paged chunked-prefill attention on gfx950 matrix cores (bf16 q, bf16 KV).
//
// Sequence b holds L cached tokens, the last C of which are this chunk's;
// query row (token i, head n) of the chunk attends to the keys at positions
// t <= p = L - C + i (causal within the chunk).  Queries are packed over
// the batch: rows q_start[b] .. q_start[b+1] of q.
//
// One workgroup of kWaves waves per (tile of COLS query rows, KV head g).
// A sequence's query rows are ordered token-major, head-minor
// (row = i * G + n), so a tile holds consecutive tokens and all G heads
// that share KV head g.  Each wave owns 16 * R of the tile's rows, as R
// column tiles of the matrix-core products
//
//   S^T[32 keys][16 rows] = K[32 keys][D] . Q^T[D][16 rows]
//   O^T[D][16 rows]      += V^T[D][32 keys] . P^T[32 keys][16 rows]
//
// (v_mfma_f32_16x16x32_bf16), with the same operand layouts as the decode
// kernel: lane (n, j) = (l % 16, l / 16) ends up owning the scores of keys
// 8j .. 8j+7 of the step for row n, which is exactly its k-slot set of
// P^T in the PV product, so P never moves between lanes.
//
// K/V go through LDS: every step (32 keys = two 16-token blocks) the whole
// workgroup copies the two K tiles ([16][D] each) and the two V tiles
// ([D][16] each) of KV head g into one of two LDS buffers, while computing
// on the other; K rows are padded by 16 bytes and V is stored as [D][32
// keys] with rows padded to 80 bytes, so the 16-byte operand reads of a
// wave hit distinct banks.  Keys at or past the sequence end, or in blocks
// with an out-of-range id, get zero V (so a masked probability times them
// is 0) and a -inf score.  The causal mask is applied only on steps that
// reach past the smallest query position of the tile.
#include <math.h>

#include "pa_launch.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kKeys = 32;  // keys per step: two blocks

template <int D>
struct PfLds {
  static constexpr int KRow = D * 2 + 16;      // bytes per K row
  static constexpr int VRow = kKeys * 2 + 16;  // bytes per V row [d][32]
  static constexpr int KBytes = kKeys * KRow;
  static constexpr int Stage = KBytes + D * VRow;
};

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Keeps the 16-bit elements e of w (8 of them) with lo <= e < hi.
__device__ __forceinline__ u32x4 keep_range(u32x4 w, int lo, int hi) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned m = (2 * k >= lo && 2 * k < hi ? 0x0000FFFFu : 0u) |
                       (2 * k + 1 >= lo && 2 * k + 1 < hi ? 0xFFFF0000u : 0u);
    w[k] &= m;
  }
  return w;
}

template <int D, int R>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k_pool,
    const __bf16* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_start, __bf16* __restrict__ out,
    PrefillSched sc) {
  typedef PfLds<D> Lay;
  constexpr int NC = D / 32;
  constexpr int NX = D / 16;
  constexpr int COLS = kPfWaves * 16 * R;
  constexpr int CPT = (8 * D) / kPfThreads;  // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Lay::Stage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int j = lane >> 4;
  const int g = blockIdx.x % sc.Hkv;
  const int tile = blockIdx.x / sc.Hkv;
  const int G = sc.G;

  // which sequence and which of its tiles (every wave finds the same)
  int b = -1, t_in_b = 0;
  {
    int carry = 0;
    for (int c0 = 0; c0 < sc.B && b < 0; c0 += kWave) {
      const int bb = c0 + lane;
      int tiles = 0;
      if (bb < sc.B) {
        int lo = q_start[bb], hi = q_start[bb + 1];
        lo = lo < 0 ? 0 : (lo > sc.T ? sc.T : lo);
        hi = hi < lo ? lo : (hi > sc.T ? sc.T : hi);
        tiles = ((hi - lo) * G + COLS - 1) / COLS;
      }
      const int incl = wave_incl_scan(tiles) + carry;
      const uint64_t hit = __ballot(bb < sc.B && tile < incl &&
                                    tile >= incl - tiles);
      if (hit) {
        const int i = __builtin_ctzll(hit);
        b = c0 + i;
        t_in_b = tile - (readlane(incl, i) - readlane(tiles, i));
      }
      carry = readlane(incl, kWave - 1);
    }
  }
  if (b < 0) return;

  int qs = q_start[b], qe = q_start[b + 1];
  qs = qs < 0 ? 0 : (qs > sc.T ? sc.T : qs);
  qe = qe < qs ? qs : (qe > sc.T ? sc.T : qe);
  const int C = qe - qs;
  const int cap = sc.max_blocks * kBlock;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int rows_b = C * G;
  const int row0 = t_in_b * COLS;
  const int nblk = (L + kBlock - 1) / kBlock;

  // rows of this wave: row0 + wave*16R + 16x + r16
  int pos[R];      // query position, -1 for a row past the chunk
  bf16x8 qb[R][NC];
#pragma unroll
  for (int x = 0; x < R; ++x) {
    const int row = row0 + wave * 16 * R + 16 * x + r16;
    const bool valid = row < rows_b;
    const int i = valid ? row / G : 0;
    const int n = valid ? row - i * G : 0;
    pos[x] = valid ? L - C + i : -1;
    const __bf16* qrow = q + ((size_t)(qs + i) * sc.Hq + (size_t)g * G + n) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qb[x][c] = valid ? *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * j)
                       : z;
    }
  }
  const int last_row = (rows_b < row0 + COLS ? rows_b : row0 + COLS) - 1;
  const int p_max = L - C + last_row / G;       // largest query position
  const int p_min = L - C + row0 / G;           // smallest
  const int kend = p_max + 1 < L ? p_max + 1 : L;  // keys needed
  const int nsteps = kend > 0 ? (kend + kKeys - 1) / kKeys : 0;

  f32x4 acc[R][NX];
  float m[R], lsum[R];
#pragma unroll
  for (int x = 0; x < R; ++x) {
    m[x] = -INFINITY;
    lsum[x] = 0.f;
#pragma unroll
    for (int X = 0; X < NX; ++X) acc[x][X] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* trow = block_tables + (size_t)b * sc.max_blocks;
  const size_t tile_elems = (size_t)kBlock * D;
  // valid keys of block blk (uniform): 0 past the end or for a bad id
  auto block_valid = [&](int blk, int id) -> int {
    if (blk >= nblk || (unsigned)id >= (unsigned)sc.NB) return 0;
    const int v = L - blk * kBlock;
    return v > kBlock ? kBlock : v;
  };

  u32x4 regs[CPT];
  int nv[2];
  auto load_stage = [&](int s) {
    int id[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int blk = 2 * s + h;
      const int raw = trow[blk < nblk ? blk : nblk - 1];
      nv[h] = block_valid(blk, raw);
      id[h] = (unsigned)raw < (unsigned)sc.NB ? raw : 0;
    }
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ch = tid + kPfThreads * u;   // [0, 8D)
      const bool is_v = ch >= 4 * D;
      const int w = is_v ? ch - 4 * D : ch;
      const int h = w / (2 * D);
      const int within = w - h * 2 * D;
      const __bf16* pool = is_v ? v_pool : k_pool;
      const __bf16* src = pool +
                          ((size_t)id[h] * sc.Hkv + g) * tile_elems +
                          (size_t)within * 8;
      regs[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* base = lds + buf * Lay::Stage;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int ch = tid + kPfThreads * u;
      const bool is_v = ch >= 4 * D;
      const int w = is_v ? ch - 4 * D : ch;
      const int h = w / (2 * D);
      const int within = w - h * 2 * D;
      if (!is_v) {
        const int key = h * kBlock + within / (D / 8);
        const int col = within % (D / 8);
        *reinterpret_cast<u32x4*>(base + key * Lay::KRow + col * 16) =
            regs[u];
      } else {
        const int d = within >> 1;
        const int half = within & 1;
        const u32x4 val = keep_range(regs[u], 0, nv[h] - 8 * half);
        *reinterpret_cast<u32x4*>(base + Lay::KBytes + d * Lay::VRow +
                                  (h * kBlock + half * 8) * 2) = val;
      }
    }
  };

  if (nsteps > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();

  // lane-constant LDS offsets of the operands
  int k_off[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int key = 16 * (r16 >> 3) + 8 * ((r16 >> 2) & 1) + 4 * s2 + (r16 & 3);
    k_off[s2] = key * Lay::KRow + 16 * j;   // + 64 c
  }
  const int v_off = Lay::KBytes + r16 * Lay::VRow + 16 * j;  // + 16X rows

  // The next stage's loads are issued unconditionally (the last step
  // reloads its own stage into the idle buffer): loads under a branch would
  // make the compiler wait for all of them before the first product.
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;
    const int nv_cur0 = nv[0], nv_cur1 = nv[1];
    load_stage(more ? s + 1 : s);
    const uint8_t* base = lds + buf * Lay::Stage;

    bf16x8 ka[2][NC];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int c = 0; c < NC; ++c)
        ka[s2][c] = *reinterpret_cast<const bf16x8*>(base + k_off[s2] +
                                                     64 * c);
    const int key0 = s * kKeys;
    const bool full = nv_cur0 == kBlock && nv_cur1 == kBlock &&
                      key0 + kKeys - 1 <= p_min;
    // this lane's 8 keys: key0 + 8j + e, valid in its block up to nvh
    const int nvh = (j < 2 ? nv_cur0 : nv_cur1) - 8 * (j & 1);
    bf16x8 pb[R];
#pragma unroll
    for (int x = 0; x < R; ++x) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s0 = mfma16x16x32(ka[0][c], qb[x][c], s0);
        s1 = mfma16x16x32(ka[1][c], qb[x][c], s1);
      }
      float xs[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[i] = s0[i] * sc.c_log2;
        xs[4 + i] = s1[i] * sc.c_log2;
      }
      if (!full) {
        const int lim = pos[x] - (key0 + 8 * j);  // e <= lim attends
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xs[e] = (e <= lim && e < nvh) ? xs[e] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])),
                       fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7])));
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m[x], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m[x] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pe = (__bf16)fast_exp2(xs[e] - m_use);
        pb[x][e] = pe;
        psum += (float)pe;
      }
      lsum[x] = lsum[x] * alpha + psum;
      m[x] = m_new;
#pragma unroll
      for (int X = 0; X < NX; ++X) acc[x][X] *= alpha;
    }
#pragma unroll
    for (int X = 0; X < NX; ++X) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(
          base + v_off + 16 * X * Lay::VRow);
#pragma unroll
      for (int x = 0; x < R; ++x) acc[x][X] = mfma16x16x32(va, pb[x], acc[x][X]);
    }
    store_stage(buf ^ 1);
    __syncthreads();
  }

  // lane (n, j) holds O[row n][16X + 4j + i]
#pragma unroll
  for (int x = 0; x < R; ++x) {
    float ltot = lsum[x] + __shfl_xor(lsum[x], 16, kWave);
    ltot += __shfl_xor(ltot, 32, kWave);
    const int row = row0 + wave * 16 * R + 16 * x + r16;
    if (row >= rows_b) continue;
    const int i = row / G;
    const int n = row - i * G;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    __bf16* orow = out + ((size_t)(qs + i) * sc.Hq + (size_t)g * G + n) * D +
                   4 * j;
#pragma unroll
    for (int X = 0; X < NX; ++X) {
      bf16x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = (__bf16)(acc[x][X][k] * inv);
      *reinterpret_cast<bf16x4*>(orow + 16 * X) = o;
    }
  }
}

template <int D, int R>
void launch_pf(const PrefillArgs& a, hipStream_t stream) {
  constexpr int COLS = kPfWaves * 16 * R;
  const int tiles = (int)(((int64_t)a.s.T * a.s.G + COLS - 1) / COLS) + a.s.B;
  hipLaunchKernelGGL((prefill_mfma_kernel<D, R>),
                     dim3((unsigned)(tiles * a.s.Hkv)), dim3(kPfThreads), 0,
                     stream, reinterpret_cast<const __bf16*>(a.q),
                     reinterpret_cast<const __bf16*>(a.k_pool),
                     reinterpret_cast<const __bf16*>(a.v_pool), a.block_tables,
                     a.seq_lens, a.q_start, reinterpret_cast<__bf16*>(a.out),
                     a.s);
}

}  // namespace

int64_t prefill_grid(int head_size, int64_t T, int G, int B, int Hkv) {
  const int cols = kPfWaves * 16 * kPrefillTiles;
  (void)head_size;
  return ((T * G + cols - 1) / cols + B) * Hkv;
}

hipError_t launch_prefill(int head_size, const PrefillArgs& a,
                          hipStream_t stream) {
  if (a.s.B == 0 || a.s.T == 0) return hipSuccess;
  switch (head_size) {
    case 64: launch_pf<64, kPrefillTiles>(a, stream); break;
    case 128: launch_pf<128, kPrefillTiles>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
