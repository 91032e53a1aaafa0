// Several products in one launch ("grouped"), for steps made of many small
// products (a layer's forward, data-gradient and weight-gradient products at
// a few thousand tokens), where a launch per product leaves most of the chip
// idle and pays a dispatch each.  One launch covers every product of one
// operand layout and format pair: its blocks are (product, 128 x 128 output
// tile, contraction slice) triples, read from a table in the kernel
// arguments.  Products with long contractions are cut into slices of about
// the group's shortest contraction, so the blocks do similar work; a split
// product's slices store raw sums in the caller's workspace, and one more
// launch adds them in slice order and unscales (the bits are the same on
// every call).  Products too large to gain (kGroupMaxTiles tiles or more:
// at least a whole wave of the single-product kernel's 256 x 256 tiles) or
// that the pipelined kernels do not take run as single products.
#pragma once

#include "gemm_split.h"

namespace fp8lin {
namespace gemm_detail {

constexpr int kGroupMax = 14;            // products per launch (kernel-argument table)
constexpr int kGroupMaxTiles = 1024;     // products this large fill the chip alone
constexpr int kGroupMinSliceStages = 8;  // shortest contraction slice of a split
constexpr int kGroupSlots = 512;         // 128 x 128 workgroups the chip runs at once (2 per CU)

// The order of a launch's products: longest blocks (most contraction stages
// per slice) first, so that the blocks handed out last are short ones.
inline void order_longest_first(const GroupSlot* plan, int* idx, int n) {
  for (int a = 1; a < n; ++a) {  // stable insertion sort by descending kslice
    const int v = idx[a];
    int b = a;
    while (b > 0 && plan[idx[b - 1]].kslice < plan[v].kslice) {
      idx[b] = idx[b - 1];
      --b;
    }
    idx[b] = v;
  }
}

struct GroupEntry {
  GemmProblem p;
  int tiles_m, tiles_n, splits, kslice, first;
  int variant;  // in the training-step kernel: which of its three products
  float* ws;    // splits > 1: slice s of the raw sums at ws + s * m * n
};

struct GroupArgs {
  int count;
  GroupEntry e[kGroupMax];
};

// The entry of the block's product: the last whose first block is at most
// blockIdx.x, read through the kernel-argument pointer (scalar loads).
template <typename Args, typename Entry>
__device__ __forceinline__ const __attribute__((address_space(4))) Entry* group_entry() {
  const auto* a = (const __attribute__((address_space(4))) Args*)__builtin_amdgcn_kernarg_segment_ptr();
  const int b = (int)blockIdx.x;
  int i = 0;
  while (i + 1 < a->count && a->e[i + 1].first <= b) ++i;
  return &a->e[i];
}

// One block's (product, tile, slice) of a grouped launch: e is its entry, sa
// and sb the block's LDS rings.
template <bool AK, bool BK, int FA, int FB, int MATH>
__device__ __forceinline__ void group_block(const __attribute__((address_space(4))) GroupEntry* e,
                                            uint8_t* sa, uint8_t* sb) {
  constexpr int R = 128;
  GemmProblem q;
  __builtin_memcpy(&q, (const GemmProblem*)&e->p, sizeof(GemmProblem));
  const int tiles_m = e->tiles_m, tiles_n = e->tiles_n, splits = e->splits, kslice = e->kslice;
  const int local = (int)blockIdx.x - e->first;
  const int tiles = tiles_m * tiles_n;
  const int s = local / tiles;
  int tm, tn;
  tile_coords(local - s * tiles, tiles_m, tiles_n, tm, tn);
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int m0 = tm * R, n0 = tn * R;

  // the slice: contraction [k0, k0 + q.k) of both operands
  const int k0 = s * kslice;
  const int ktot = q.k;
  q.k = min(kslice, ktot - k0);
  q.a += AK ? (int64_t)k0 : (int64_t)k0 * q.lda;
  q.b += BK ? (int64_t)k0 : (int64_t)k0 * q.ldb;

  v16f acc[2][2];
  zero_acc(acc);
  QuadWave<AK, BK, FA, FB, MATH> w(q, m0, n0, wave, lane, lds_addr(sa), lds_addr(sb), acc);
  w.run();
  const int row0 = m0 + (wave >> 1) * (R / 2), col0 = n0 + (wave & 1) * (R / 2);
  if (splits == 1) store_block_as<false>(q, acc, row0, col0, lane);
  else store_raw_block(e->ws + (int64_t)s * q.m * q.n, q.m, q.n, acc, row0, col0, lane);
}

template <bool AK, bool BK, int FA, int FB, int MATH>
__global__ __launch_bounds__(256) void gemm_group_kernel(GroupArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t sa[kPipeStages * 128 * kPipeBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sb[kPipeStages * 128 * kPipeBK];
  group_block<AK, BK, FA, FB, MATH>(group_entry<GroupArgs, GroupEntry>(), sa, sb);
}

// The ordered sum of the split products' slices: out[i] = 2^-(ba+bb) *
// (ws[i] + ws[mn + i] + ...), the products' own unscale once at the end.
struct ReduceEntry {
  const float* ws;
  float* out;
  const int32_t* bias_a;
  const int32_t* bias_b;
  int64_t mn;
  int splits, first, blocks, vec;
};

struct ReduceArgs {
  int count;
  ReduceEntry e[kGroupMax];
};

// (A template so that every layout's translation unit can instantiate it.)
template <int kUnused>
__global__ __launch_bounds__(kReduceThreads) void group_reduce_kernel(ReduceArgs args) {
  const auto* e = group_entry<ReduceArgs, ReduceEntry>();
  const float* __restrict__ ws = e->ws;
  float* __restrict__ out = e->out;
  const int unscale = -(*e->bias_a + *e->bias_b);
  const int splits = e->splits;
  const int64_t mn = e->mn;
  const int64_t stride = (int64_t)e->blocks * kReduceThreads;
  const int64_t first = ((int64_t)blockIdx.x - e->first) * kReduceThreads + threadIdx.x;
  if (e->vec) {
    const int64_t n4 = mn / 4;
    const float4* w4 = reinterpret_cast<const float4*>(ws);
    float4* o4 = reinterpret_cast<float4*>(out);
    for (int64_t i = first; i < n4; i += stride) {
      float4 acc = w4[i];
      for (int sl = 1; sl < splits; ++sl) {
        const float4 v = w4[(int64_t)sl * n4 + i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
      o4[i] = make_float4(__builtin_ldexpf(acc.x, unscale), __builtin_ldexpf(acc.y, unscale),
                          __builtin_ldexpf(acc.z, unscale), __builtin_ldexpf(acc.w, unscale));
    }
  } else {
    for (int64_t i = first; i < mn; i += stride) {
      float acc = ws[i];
      for (int sl = 1; sl < splits; ++sl) acc += ws[(int64_t)sl * mn + i];
      out[i] = __builtin_ldexpf(acc, unscale);
    }
  }
}

// One launch (or a few, kGroupMax products at a time) of the products ps[idx[j]]
// (all of layout AK, BK and formats FA, FB), then the reduction of the split ones.
template <bool AK, bool BK, int FA, int FB, int MATH>
hipError_t launch_group_bucket(const GemmProblem* ps, const GroupSlot* plan, const int* idx_in, int n,
                               uint8_t* ws, hipStream_t stream) {
  int idx[kGroupMaxProducts];
  for (int j = 0; j < n; ++j) idx[j] = idx_in[j];
  order_longest_first(plan, idx, n);
  for (int lo = 0; lo < n; lo += kGroupMax) {
    const int cnt = n - lo < kGroupMax ? n - lo : kGroupMax;
    GroupArgs g{};
    ReduceArgs r{};
    g.count = cnt;
    int64_t blocks = 0, rblocks = 0;
    for (int j = 0; j < cnt; ++j) {
      const GemmProblem& p = ps[idx[lo + j]];
      const GroupSlot& sl = plan[idx[lo + j]];
      GroupEntry& e = g.e[j];
      e.p = p;
      e.p.amax = nullptr;
      e.tiles_m = (p.m + 127) / 128;
      e.tiles_n = (p.n + 127) / 128;
      e.splits = sl.splits;
      e.kslice = sl.kslice;
      e.first = (int)blocks;
      e.ws = sl.splits > 1 ? reinterpret_cast<float*>(ws + sl.ws_offset) : nullptr;
      blocks += (int64_t)e.tiles_m * e.tiles_n * e.splits;
      if (sl.splits > 1) {
        ReduceEntry& q = r.e[r.count++];
        const int64_t mn = (int64_t)p.m * p.n;
        const bool vec = (mn & 3) == 0;
        const int64_t units = vec ? mn / 4 : mn;
        int64_t b = (units + kReduceThreads - 1) / kReduceThreads;
        b = b < 1 ? 1 : (b > 2048 ? 2048 : b);
        q = ReduceEntry{e.ws, p.c, p.bias_a, p.bias_b, mn, sl.splits, (int)rblocks, (int)b, vec ? 1 : 0};
        rblocks += b;
      }
    }
    hipLaunchKernelGGL((gemm_group_kernel<AK, BK, FA, FB, MATH>), dim3((uint32_t)blocks), dim3(256), 0,
                       stream, g);
    if (hipError_t err = hipGetLastError()) return err;
    if (r.count > 0) {
      hipLaunchKernelGGL(group_reduce_kernel<0>, dim3((uint32_t)rblocks), dim3(kReduceThreads), 0, stream, r);
      if (hipError_t err = hipGetLastError()) return err;
    }
  }
  return hipSuccess;
}

template <bool AK, bool BK, int MATH>
hipError_t launch_group_math(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                             uint8_t* ws, hipStream_t stream) {
  // sub-buckets by format pair
  int sub[4][kGroupMaxProducts];
  int cnt[4] = {0, 0, 0, 0};
  for (int j = 0; j < n; ++j) {
    const GemmProblem& p = ps[idx[j]];
    const int k = (p.fmt_a == FP8_E5M2 ? 1 : 0) + (p.fmt_b == FP8_E5M2 ? 2 : 0);
    sub[k][cnt[k]++] = idx[j];
  }
  if (cnt[0]) if (hipError_t e = launch_group_bucket<AK, BK, FP8_E4M3, FP8_E4M3, MATH>(ps, plan, sub[0], cnt[0], ws, stream)) return e;
  if (cnt[1]) if (hipError_t e = launch_group_bucket<AK, BK, FP8_E5M2, FP8_E4M3, MATH>(ps, plan, sub[1], cnt[1], ws, stream)) return e;
  if (cnt[2]) if (hipError_t e = launch_group_bucket<AK, BK, FP8_E4M3, FP8_E5M2, MATH>(ps, plan, sub[2], cnt[2], ws, stream)) return e;
  if (cnt[3]) if (hipError_t e = launch_group_bucket<AK, BK, FP8_E5M2, FP8_E5M2, MATH>(ps, plan, sub[3], cnt[3], ws, stream)) return e;
  return hipSuccess;
}

// Every grouped product of one layout (idx: their indices into ps / plan).
// The exact arithmetic's MFMA follows the formats, as for single products
// (bf16 when an operand is E5M2, fp16 otherwise), so each format pair's
// bucket takes its own arithmetic.
template <bool AK, bool BK>
hipError_t launch_group_layout(const GemmProblem* ps, const GroupSlot* plan, const int* idx, int n,
                               uint8_t* ws, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (ps[idx[0]].math == kMathNativeFp8) return launch_group_math<AK, BK, kMathNativeFp8>(ps, plan, idx, n, ws, stream);
  int f16[kGroupMaxProducts], bf16[kGroupMaxProducts];
  int nf = 0, nb = 0;
  for (int j = 0; j < n; ++j) {
    if (exact_on_bf16(ps[idx[j]])) bf16[nb++] = idx[j];
    else f16[nf++] = idx[j];
  }
  if (nf) if (hipError_t e = launch_group_math<AK, BK, kMathExact>(ps, plan, f16, nf, ws, stream)) return e;
  if (nb) if (hipError_t e = launch_group_math<AK, BK, kMathExactBf16>(ps, plan, bf16, nb, ws, stream)) return e;
  return hipSuccess;
}

}  // namespace gemm_detail
}  // namespace fp8lin
