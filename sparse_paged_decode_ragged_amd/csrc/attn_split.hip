// attn_split.hip -- split-L sparse decode attention with the partitions
// merged inside the same kernel, gfx950.
//
// Operation (sglang PR #28392 summary page, "key source snippet": the
// paged_decode.py module docstring): token t attends to the pool rows
// kv_indices[kv_indptr[t] : kv_indptr[t+1]]; each bf16 row is both key and
// value; attn_sink[H] is a virtual key of the softmax denominator; online
// softmax in the log2 domain; an empty slice gives zeros.  Cutting a long
// slice into partitions whose (m, l, O) states are merged afterwards is the
// split-L plus combine design of the same path.
//
// Why this decomposition.  A small decode batch (tens of tokens, 64 heads,
// D = 512) gives one workgroup per (token, head group) for a fraction of the
// chip, and spreading the heads over several workgroups pulls every gathered
// row into several CUs.  Here a workgroup is (token, 32 HB heads, partition c
// of R rows): every gathered row enters one CU (HB = 2: 64 heads) or two (HB
// = 1, two head groups of a token), and each CU's rows are a quarter or half
// of what a head-split workgroup would take in.  R is either fixed by the
// host (split_rows; grid N x head groups x splits) or chosen by the kernel
// from the call's slice lengths (balanced plans: 256 workgroups dealt out as
// the partitions of all slices, token by token), so that a long slice among
// short ones takes more of the chip.
//
// Inside a workgroup: 4 waves of 32 heads (two 16-head MFMA blocks per wave,
// as in the 32-head-wave heads kernel): HB head blocks x P parities.  A
// super-tile of 16 P rows sits in an LDS ring (LDS-DMA gathers, XOR-swizzled
// rows); wave (hb, par) computes heads 32 hb .. of rows [16 par, 16 par + 16):
//   S^T = K Q^T on 16x16x32 MFMAs (one K read feeds both head blocks),
//   O^T += V^T P^T on 32x32x16 MFMAs over the 16 rows (P^T from the two
//   blocks' weights after one v_permlane16_swap per dword),
// so each K and V^T byte read from LDS feeds 32 heads.  At the end the P
// parity states of a head block merge in LDS (a butterfly over the parities),
// leaving each wave the merged state of its 32 heads on D / P columns: the
// wave's piece.
//
// Merging the partitions without a second launch.  Each of the four pieces
// of a (token, head group) is cut into U units of whole d-tiles, U the least
// power of two with 4 U >= nparts, and unit u of the 4 U is merged by
// partition u mod nparts (a reduce-scatter: every partition merges a share).  Every partition publishes its pieces to the workspace with
// agent-scope coherent stores (sc1), waits until the stores are complete and
// counts itself in with one atomic add on each unit another partition merges;
// the merging workgroup polls the unit's counter (read-modify-writes at agent
// scope), then reads every partition's share of the unit (sc1 loads), sums
// them in partition order (every arrival order gives the same bits), writes
// the output and resets the counter to zero.  It waits only when the whole
// grid fits on the chip at once (one workgroup per CU), and then for a bounded
// time: past the bound, or at once on a larger grid, it counts itself in as
// well, and whichever arrival completes the count merges instead -- so no wave
// ever waits on a workgroup that cannot be scheduled.  No whole-cache
// write-back or invalidation is involved: only these sc1 accesses carry data
// between workgroups, and an sc1 load is served at agent scope, never from a
// line an XCD's L2 kept from before the publishing stores.
//
// FP8 rows (kFp8): the same kernel over D code bytes a row with an fp32 scale
// a row (sglang PR #25898 summary page, "key files": the FP8 caches), the
// codes decoded to bf16 exactly before each MFMA and the scale applied to the
// row's scores and weights, as in attn_fp8.hip.
#include <atomic>

#include "fp8_device.h"

namespace spd {
namespace {

constexpr int kSplitIdx = 1024;  // row indices staged at a time
// A merging workgroup waits for its partners at most this long, on the 100
// MHz real-time counter: partners of equal length that are resident arrive
// within a few microseconds; one that is not (a kernel on another stream
// holding CUs) is not waited for past the bound.  A partition shorter than
// the others of its slice (its last one) waits besides for the rows it lacks,
// at kSpinTicksPerRow a row (a resident workgroup takes about 0.07 us a row),
// up to kSpinTicksMax: giving up earlier leaves its units to the last arrival,
// which merges them one wave at a time (ragged batch in a balanced plan: 107
// us with a flat 20 us bound, 87 us with the longer one).
constexpr uint64_t kSpinTicks = 2000;        // 20 us
constexpr uint64_t kSpinTicksPerRow = 10;    // 0.1 us
constexpr uint64_t kSpinTicksMax = 100000;   // 1 ms
constexpr int kSpinLimit = 1 << 20;  // polls (the time bound ends the wait first)

// Balanced plans: a head group's bal_slots workgroups are the partitions of
// the call's slices, numbered token by token.  K, the least number of
// super-tiles for which ceil(lk / K) partitions of every slice (lk its
// super-tiles) fit, and at least the longest slice's over kBalMaxParts, sets
// the partition counts; a split slice's super-tiles are then shared evenly
// by its partitions (ceil(lk / count) each, at most K, the last taking the
// rest).  Each wave derives the plan and its workgroup's (token, partition)
// from kv_indptr alone, so the grid stays fixed by the host while the split
// follows this call's lengths.
constexpr int kBalPer = 8;        // tokens a lane holds (N <= 512)
constexpr int kBalMaxParts = 32;  // partitions of one slice (the merge's units)

// ceil(a / b) for 0 <= a < 2^31, b >= 1 and a / b <= 32, with rb = 1 / b in
// fp32: the product is within 2^-16 of a / b, so its truncation lies at most
// two below the ceiling, which the two integer steps reach exactly (q b stays
// below 2^32).
__device__ __forceinline__ int ceil_div_small(int a, int b, float rb) {
  unsigned q = (unsigned)((float)a * rb);
  q += q * (unsigned)b < (unsigned)a ? 1u : 0u;
  q += q * (unsigned)b < (unsigned)a ? 1u : 0u;
  return (int)q;
}

// Sum or maximum over the wave, in every lane: DPP steps within rows of 16
// lanes, then the two halves and the two quarters swapped across (VALU only,
// no LDS round trips).
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}

template <bool kMax>
__device__ __forceinline__ int wave_reduce_i(int v) {
  auto op = [](int a, int b) { return kMax ? max(a, b) : a + b; };
  v = op(v, dpp_i<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_i<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_i<0x141>(v));  // row_half_mirror
  v = op(v, dpp_i<0x140>(v));  // row_mirror
  const auto a = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  v = op((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  return op((int)b[0], (int)b[1]);
}

struct BalancedItem {
  bool zero_j; // slice j (j < N) is empty: this workgroup writes its zeros
  int t;       // token, or -1 when the partitions end before this workgroup
  int c;       // partition of the token
  int nparts;  // partitions of the token's slice
  int row0;    // kv_indptr[t]
  int L;       // rows of the slice
  int R;       // rows of each partition but the slice's last (which takes the rest)
};

// The kv_indptr entries lane l holds for a balanced plan over N <= 64 kBalPer
// slices: tokens [l per, l per + per), per = ceil(N / 64).
__device__ __forceinline__ void balanced_load(const int32_t* indptr, int N, int lane,
                                              int (&st)[kBalPer + 1]) {
  const int t0 = lane * ((N + 63) >> 6);
#pragma unroll
  for (int i = 0; i <= kBalPer; ++i) st[i] = indptr[t0 + i < N ? t0 + i : N];
}

// Item j (< slots) of a balanced plan over the N <= 64 kBalPer slices whose
// kv_indptr entries balanced_load gave (slots >= N, so one partition a slice
// always fits).  The result is wave-uniform.
template <int kSuper>
__device__ __forceinline__ BalancedItem balanced_item(const int (&st)[kBalPer + 1], int N,
                                                      int slots, int j, int lane) {
  static_assert((kSuper & (kSuper - 1)) == 0, "super-tile rows: a power of two");
  const int per = (N + 63) >> 6;
  const int t0 = lane * per;
  int lk[kBalPer];  // super-tiles of each slice
  int mx = 0, sum = 0, nz = 0, lj = 0;
#pragma unroll
  for (int i = 0; i < kBalPer; ++i) {
    const int L = i < per && t0 + i < N ? st[i + 1] - st[i] : 0;
    lk[i] = L > 0 ? (L - 1) / kSuper + 1 : 0;
    mx = max(mx, lk[i]);
    sum += lk[i];
    nz += lk[i] > 0 ? 1 : 0;
    lj = t0 + i == j ? lk[i] : lj;  // (in the lane holding token j)
  }
  const bool zero_j = j < N && __builtin_amdgcn_readlane(lj, j < N ? j / per : 0) == 0;
  // (the wave sums are uniform; readfirstlane tells the compiler so, which
  // keeps the search and everything sized by its result in scalar registers)
  mx = __builtin_amdgcn_readfirstlane(wave_reduce_i<true>(mx));
  BalancedItem r{zero_j, -1, 0, 0, 0, 0, kSuper};
  if (mx == 0) return r;  // every slice empty
  const int S = __builtin_amdgcn_readfirstlane(wave_reduce_i<false>(sum));  // <= 2^26 + N
  const int n = __builtin_amdgcn_readfirstlane(wave_reduce_i<false>(nz));
  // least k (super-tiles a partition) of at least mx / kBalMaxParts whose
  // partitions fit.  The count sum_t ceil(lk_t / k) falls as k grows and lies
  // in [S / k, S / k + n], so it fits from some k in [S / slots, S / (slots -
  // n)], and at k = mx (one partition a slice)
  int klo = (mx + kBalMaxParts - 1) / kBalMaxParts, khi = mx;
  klo = max(klo, (S + slots - 1) / slots);
  if (slots > n) khi = min(khi, max(klo, (S + (slots - n) - 1) / (slots - n)));
  klo = min(klo, khi);
  while (klo < khi) {
    const int mid = (klo + khi) >> 1;
    const float rm = 1.0f / (float)mid;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kBalPer; ++i)
      if (i < per) cnt += ceil_div_small(lk[i], mid, rm);
    cnt = __builtin_amdgcn_readfirstlane(wave_reduce_i<false>(cnt));
    if (cnt <= slots)
      khi = mid;
    else
      klo = mid + 1;
  }
  const float rk = 1.0f / (float)klo;
  int np[kBalPer];
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kBalPer; ++i) {
    np[i] = i < per ? ceil_div_small(lk[i], klo, rk) : 0;
    tot += np[i];
  }
  int incl = tot;  // partitions of lanes 0 .. lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  int pre = incl - tot;
  bool found = false;
  int ft = 0, fc = 0, fnp = 0, frow0 = 0, fL = 0, flk = 0;
#pragma unroll
  for (int i = 0; i < kBalPer; ++i) {
    if (!found && j >= pre && j < pre + np[i]) {
      found = true;
      ft = t0 + i;
      fc = j - pre;
      fnp = np[i];
      frow0 = st[i];
      fL = st[i + 1] - st[i];
      flk = lk[i];
    }
    pre += np[i];
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(found);
  if (m == 0) return r;
  const int f = __builtin_ctzll(m);
  r.t = __builtin_amdgcn_readlane(ft, f);
  r.c = __builtin_amdgcn_readlane(fc, f);
  r.nparts = __builtin_amdgcn_readlane(fnp, f);
  r.row0 = __builtin_amdgcn_readlane(frow0, f);
  r.L = __builtin_amdgcn_readlane(fL, f);
  // a split slice's partitions share its super-tiles evenly (at most klo
  // each), so that a partition that also merges does not take the longest
  // share of rows as well
  const int lkf = __builtin_amdgcn_readlane(flk, f);
  r.R = (r.nparts > 1 ? (lkf + r.nparts - 1) / r.nparts : klo) * kSuper;
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base) {
  // raw buffer over a piece's slot (< 2 GiB), untyped 32-bit format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

constexpr int kSc1 = 16;  // cache policy bit of an agent-scope coherent access

// Four accumulator values as four bf16 (round to nearest even), stored and
// loaded as 8 bytes; the load widens them back to fp32 exactly.
__device__ __forceinline__ void store_bf16x4_sc1(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4 load_bf16x4_sc1(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, kSc1);
  return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xffff0000u),
               __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xffff0000u)};
}
__device__ __forceinline__ void store1_sc1(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, kSc1);
}
__device__ __forceinline__ float load1_sc1(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, kSc1));
}

// Weight 2^(m - M) of a state with reference maximum m in a merge whose
// maximum is M >= m; a state that saw no row (m = -inf) weighs exactly 0, also
// when every merged state is empty (M = -inf, where 2^(m - M) would be NaN).
__device__ __forceinline__ float state_weight(float m, float M) {
  return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
}

__device__ __forceinline__ f32x4 quarter(const f32x16& v, int e4) {
  return f32x4{v[4 * e4], v[4 * e4 + 1], v[4 * e4 + 2], v[4 * e4 + 3]};
}

__device__ __forceinline__ void set_quarter(f32x16& v, int e4, f32x4 q) {
  v[4 * e4] = q[0];
  v[4 * e4 + 1] = q[1];
  v[4 * e4 + 2] = q[2];
  v[4 * e4 + 3] = q[3];
}

// A piece's slot in the workspace: its kDTw d-tiles as the register image of
// the accumulators in bf16 (each f32x16 stored as four 8-byte columns of 64
// lanes), then m of its 32 heads, then l, both fp32.  Exchanging O in bf16
// halves the bytes that go through memory between the partitions; it adds
// one rounding (2^-9 relative) to each partition's unnormalised O, while m
// and l, which set the weights, stay exact.
template <int D, int P>
struct Piece {
  static constexpr int kDTw = D / 32 / P;
  static constexpr int kOBytes = kDTw * 4 * 64 * 8;
  static constexpr int kBytes = kOBytes + 2 * 32 * 4;
};

template <int D, int HB, int P, bool kFp8>
__global__ void __launch_bounds__(256) attn_split_kernel(AttnArgs a) {
  constexpr int kWaves = 4;
  static_assert(HB * P == kWaves, "four waves: head blocks x parities");
  static_assert(!kFp8 || D >= 128, "FP8 rows: D >= 128");
  constexpr int kHeads = 32 * HB;
  constexpr int kRowBytes = kFp8 ? D : 2 * D;  // a gathered row: D codes, or D bf16
  constexpr int kQRowBytes = 2 * D;            // a row of q (bf16)
  constexpr int kSuper = 16 * P;  // rows per super-tile
  constexpr int kStageBytes = kSuper * kRowBytes;
  constexpr int kKSteps = D / 32;
  constexpr int kDT = D / 32;    // 32-wide d-tiles of the PV product
  constexpr int kDTw = kDT / P;  // d-tiles of this wave's piece
  constexpr int kRowsPerLoad = 1024 / kRowBytes;
  constexpr int kLoadsPerStage = kSuper / kRowsPerLoad;
  constexpr int kLoadsPerWave = kLoadsPerStage / kWaves;
  constexpr int kRowsPerWave = kSuper / kWaves;  // rows (and FP8 scales) a wave loads
  constexpr int kPerTile = kLoadsPerWave + (kFp8 ? 1 : 0);  // with the scales' load
  constexpr int kRing = 128 * 1024;
  // stages of the ring: what kRing holds, at most 4 bf16 or 8 FP8 super-tiles
  // (the same bytes), and no more loads in flight per wave than the 6-bit
  // vmcnt counts
  constexpr int kMaxStages = kFp8 ? 8 : 4;
  constexpr int kFit = kRing / kStageBytes < kMaxStages ? kRing / kStageBytes : kMaxStages;
  constexpr int kCount = 63 / kPerTile;
  constexpr int kStages0 = kFit < kCount ? kFit : kCount;
  constexpr int kStages = kStages0 < 2 ? 2 : kStages0;
  using Pc = Piece<D, P>;
  // LDS read lead of the QK (k-steps) and PV (d-tiles) loops
  constexpr int kKA = 2, kVA = 2;
  // super-tiles in flight when the loop starts (FP8: twice as many, the same bytes)
  constexpr int kBurstWant = kFp8 ? 4 : 2;
  constexpr int kBurst = kBurstWant < kStages ? kBurstWant : kStages;
  static_assert(D % 64 == 0 && D <= 512, "unsupported D");
  static_assert(kDTw >= 1, "a piece holds at least one d-tile");
  static_assert(kLoadsPerStage % kWaves == 0, "loads must divide among waves");
  static_assert(kStages * kPerTile <= 63, "outstanding loads must fit vmcnt");
  static_assert(kBurst <= 4, "wait_outstanding counts up to three later super-tiles");
  static_assert(P == 1 || kStages * kStageBytes >= kWaves * (kDT / 2) * 64 * 64,
                "the parity exchange reuses the ring");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
  __shared__ __attribute__((aligned(256))) int sidx[kSplitIdx];
  __shared__ __attribute__((aligned(256))) float ssink[64];
  __shared__ __attribute__((aligned(256))) float sscale[kFp8 ? kStages : 1][kWaves][64];
  __shared__ float sml[kWaves][4][16];  // per wave: m0, m1, l0, l1 of its 32 heads
  __shared__ int sflag[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hb = wave / P;
  const int par = wave % P;
  const int n16 = lane & 15;
  const int g = lane >> 4;

  // q of the workgroup's heads is staged once into the last kQStages stages of
  // the ring (rows XOR-swizzled like the tiles, so that the Q^T reads below
  // put 16 heads' same chunk in 16 bank groups), read into registers, and the
  // stages are handed back to the row tiles; rows of heads past H repeat a
  // valid row.  Its loads go out with the sinks as soon as the token is known:
  // in a fixed plan first of all, so that their latency overlaps the
  // kv_indptr and index round trips.
  constexpr int kQBytes = kHeads * kQRowBytes;
  constexpr int kQStages = (kQBytes + kStageBytes - 1) / kStageBytes;
  static_assert(kQStages < kStages, "q staging must leave a stage for the first tiles");
  constexpr int kQLoads = kQBytes / 1024;
  static_assert(kQLoads % kWaves == 0, "q loads must divide among waves");
  constexpr int kQLoadsPerWave = kQLoads / kWaves;
  unsigned char* sq = smem + (kStages - kQStages) * kStageBytes;
  auto issue_q = [&](int t, int hg) {
    constexpr int kRowsPerLd = 1024 / kQRowBytes;
    constexpr int kChunksQ = kQRowBytes / 16;
    const unsigned char* qb = reinterpret_cast<const unsigned char*>(a.q);
    const int64_t qrow0 = (int64_t)t * a.H + hg * kHeads;
#pragma unroll
    for (int k = 0; k < kQLoadsPerWave; ++k) {
      const int ld = k * kWaves + wave;
      const int r = ld * kRowsPerLd + lane / kChunksQ;  // head row within the group
      const int hr = hg * kHeads + r < a.H ? r : 0;
      const int chunk = (lane % kChunksQ) ^ (row_swizzle(r) & (kChunksQ - 1));
      dma_16B(qb + ((qrow0 + hr) * kQRowBytes + chunk * 16),
              __builtin_amdgcn_readfirstlane(lds_addr(sq + ld * 1024)));
    }
    if (wave == 0) {
      const int hs = hg * kHeads + lane;
      dma_4B(a.sink + (hs < a.H ? hs : a.H - 1), __builtin_amdgcn_readfirstlane(lds_addr(ssink)));
    }
  };

  // Work item (token, head group, partition).  Fixed plans: partition
  // fastest, then head group, so the partitions and head groups of a token
  // are consecutive items, which xcd_item keeps on one XCD (one L2) and
  // dispatches together.  Balanced plans: head group slowest, then the
  // partitions token by token (consecutive again).
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
  int t, hg, c, nparts, row0, L, R;
  int tq = -1;  // balanced plans: the token whose q went out before the plan was known
  // balanced plans: the kv_indices offset and count of the indices staged
  // before the plan was known (-1: none)
  int spec_row = -1, spec_n = 0;
  if (a.bal_slots > 0) {
    hg = item / a.bal_slots;
    const int j = item - hg * a.bal_slots;
    // A guess, so that equal slices do not wait for the plan: the token of
    // item j if every slice took the same number of partitions, and the
    // partition item j would be if every slice had the length of slice tq
    // (the plan's choice for equal slices; it lies inside slice tq).  It
    // holds only if the slices before tq are as long as tq's, which a
    // padded, ragged or skewed batch rarely gives, so q and the partition's
    // indices go out after that check (one scalar round trip, beside the
    // plan's loads) and are kept when the plan agrees; when the check fails
    // q goes out with the indices once the plan is known.
    const int each = min(kBalMaxParts, max(1, a.bal_slots / a.N));
    tq = min(j / each, a.N - 1);
    int st[kBalPer + 1];  // (the plan's loads, in flight with the guess's)
    balanced_load(a.kv_indptr, a.N, lane, st);
    {
      const int r0 = indptr[tq], lq = indptr[tq + 1] - r0;
      const int lkq = lq > 0 ? (lq - 1) / kSuper + 1 : 0;
      const int kg = (lkq + each - 1) / each;
      const int pg = kg > 0 ? (lkq + kg - 1) / kg : 0;
      const int cg = j - tq * each;
      if (lkq > 0 && pg == each && cg >= 0 && cg < pg && (int64_t)r0 == (int64_t)tq * lq) {
        issue_q(tq, hg);
        const int rg = (pg > 1 ? (lkq + pg - 1) / pg : kg) * kSuper, cbg = cg * rg;
        const int ng = cg == pg - 1 ? lq - cbg : rg;
        spec_row = r0 + cbg;
        spec_n = ng < kSplitIdx ? ng : kSplitIdx;
        stage_indices(a.kv_indices + spec_row, 0, spec_n, sidx, wave, kWaves, lane);
      } else {
        tq = -1;  // no q went out
      }
    }
    const BalancedItem b = balanced_item<kSuper>(st, a.N, a.bal_slots, j, lane);
    // an empty slice t gets its zeros from workgroup t of the head group
    // (bal_slots >= N)
    if (b.zero_j && par == 0) {
      const int hz = hg * kHeads + hb * 32;
      zero_heads<D>(a.out, a.H, j, hz, a.H - hz < 32 ? a.H - hz : 32, lane, 64);
    }
    if (b.t < 0) {  // no partition left for this workgroup
      wait_vmcnt<0>();  // no LDS-DMA load may outlive the workgroup
      return;
    }
    t = b.t;
    c = b.c;
    nparts = b.nparts;
    row0 = b.row0;
    L = b.L;
    R = b.R;
    if (tq < 0) {  // nothing was guessed: q goes out now, beside the indices
      issue_q(t, hg);
      tq = t;
    }
  } else {
    c = item % a.splits;
    const int th0 = item / a.splits;
    hg = th0 % a.head_groups;
    t = th0 / a.head_groups;
    issue_q(t, hg);
    row0 = indptr[t];
    L = indptr[t + 1] - row0;
    nparts = partitions_of(L, a.splits, a.split_rows);
    R = a.split_rows;
    if (c >= nparts || L <= 0) {
      wait_vmcnt<0>();  // no LDS-DMA load may outlive the workgroup
      // partition 0 of an empty slice: zeros
      const int hz = hg * kHeads + hb * 32;
      if (c == 0 && L <= 0 && par == 0)
        zero_heads<D>(a.out, a.H, t, hz, a.H - hz < 32 ? a.H - hz : 32, lane, 64);
      return;
    }
  }
  const int th = t * a.head_groups + hg;
  const int h0 = hg * kHeads + hb * 32;  // first head of this wave (32 heads)
  const int cb = c * R;
  const int nrows = (c == nparts - 1) ? L - cb : R;
  const int short_rows = R - nrows;  // > 0 for a slice's shorter last partition
  const int32_t* part = a.kv_indices + row0 + cb;

  // LDS read offsets of the K and V^T operands: bf16 tiles in the wide
  // swizzle, FP8 tiles in the row swizzle (one set is dead code)
  const TileOffsets<D, 1> off(n16, g);
  const WideVtOffsets<D> voff(lane);
  const Fp8KOffsets<D> off8(n16, g);
  const Fp8WideVtOffsets<D> voff8(lane);

  // wait until at most `tiles` (< kStages) later super-tiles of this wave are in flight
  auto wait_outstanding = [](int tiles) {
    constexpr int k2 = kStages > 2 ? 2 : 1, k3 = kStages > 3 ? 3 : k2;
    switch (tiles) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<kPerTile>(); break;
      case 2: wait_vmcnt<k2 * kPerTile>(); break;
      default: wait_vmcnt<k3 * kPerTile>(); break;
    }
  };

  // This wave's rows of super-tile `tile` of a chunk of n staged indices;
  // FP8: then their scales (lane l loads the scale of row l % kRowsPerWave of
  // the wave's part; positions past n repeat the last row).
  auto issue_super = [&](int n, int tile) {
    const int p0 = tile * kSuper + wave * kRowsPerWave;
    unsigned char* dst = smem + (tile % kStages) * kStageBytes + wave * kLoadsPerWave * 1024;
    if constexpr (kFp8) {
      issue_rows<kRowBytes, kLoadsPerWave>(reinterpret_cast<const uint16_t*>(a.kv8), sidx, n, p0,
                                           wave * kRowsPerWave, dst, lane);
      const int p = p0 + lane % kRowsPerWave;
      const int grow = sidx[p < n ? p : n - 1];
      dma_4B(a.kv_scale + grow,
             __builtin_amdgcn_readfirstlane(lds_addr(sscale[tile % (kFp8 ? kStages : 1)][wave])));
    } else {
      issue_rows<kRowBytes, kLoadsPerWave, 1>(a.kv, sidx, n, p0, wave * kRowsPerWave, dst, lane);
    }
  };

  // The first chunk's indices; once they (and q, issued before them) are in,
  // the first tiles go out into the stages q does not use, then q is read.
  const int n0 = nrows < kSplitIdx ? nrows : kSplitIdx;
  const int ntiles0 = (n0 + kSuper - 1) / kSuper;
  const int burst0 = ntiles0 < kBurst ? ntiles0 : kBurst;  // tiles in flight before the loop
  const int pre = burst0 < kStages - kQStages ? burst0 : kStages - kQStages;
  auto issue_tile0 = [&](int tile) { issue_super(n0, tile); };
  if (spec_row != row0 + cb || spec_n != n0) {
    if (spec_row >= 0) {  // staged for a wrong guess: those loads land before the restaging
      wait_vmcnt<0>();
      barrier_lds();
    }
    stage_indices(part, 0, n0, sidx, wave, kWaves, lane);
  }
  // (balanced plans) a wrong guess: each wave's guessed q loads land before
  // it loads the right q into the same LDS bytes; the first tiles then go out
  // before that q has landed, and q is waited for before its LDS copy is read
  const bool q_late = a.bal_slots > 0 && t != tq;
  wait_vmcnt<0>();
  if (q_late) issue_q(t, hg);
  barrier_lds();
  for (int k = 0; k < pre; ++k) issue_tile0(k);
  if (q_late) {  // every wave's share of q has landed before any wave reads it
    wait_outstanding(pre);
    barrier_lds();
  }
  bf16x8 q0[kKSteps], q1[kKSteps];  // Q^T operands of head blocks 0 and 1
  {
    // lane (n16, g) of the k-step u operand holds q[h, 32 u + 8 g .. +7]:
    // logical chunk 4 u + g of head row h, stored at chunk ^ swizzle(h)
    const int r0 = hb * 32 + n16, r1 = r0 + 16;
    constexpr int kChunksQ = kQRowBytes / 16;
    const int sw = row_swizzle(n16) & (kChunksQ - 1);  // r0 & 15 == r1 & 15 == n16
#pragma unroll
    for (int u = 0; u < kKSteps; ++u) {
      const int ch = ((4 * u + g) ^ sw) * 16;
      q0[u] = *reinterpret_cast<const bf16x8*>(sq + r0 * kQRowBytes + ch);
      q1[u] = *reinterpret_cast<const bf16x8*>(sq + r1 * kQRowBytes + ch);
    }
    barrier_lds();  // every wave has its q: the stages go back to the tiles
    for (int k = pre; k < burst0; ++k) issue_tile0(k);
  }
  float m0 = -INFINITY, l0 = 0.f, mt0 = -INFINITY, sk0 = -INFINITY;
  float m1 = -INFINITY, l1 = 0.f, mt1 = -INFINITY, sk1 = -INFINITY;
  f32x16 acc[kDT];
  for (int pass = 0; pass < 2; ++pass) {
    bool first0 = pass == 0, first1 = pass == 0;
    if (pass == 1) {
      second_pass_state(sk0, mt0, g, m0, l0);
      second_pass_state(sk1, mt1, g, m1, l1);
    }
#pragma unroll
    for (int i = 0; i < kDT; ++i) acc[i] = f32x16{};
    bool over = false;

    for (int sc = 0; sc < nrows; sc += kSplitIdx) {
      const int n = nrows - sc < kSplitIdx ? nrows - sc : kSplitIdx;
      if (sc > 0 || pass > 0) barrier_lds();  // every wave is done with the ring and indices
      if (sc > 0 || pass > 0) {
        stage_indices(part, sc, n, sidx, wave, kWaves, lane);
        wait_vmcnt<0>();
        barrier_lds();
      }
      if (pass == 0 && sc == 0) {  // the sink belongs to partition 0, parity 0
        const bool own = c == 0 && par == 0;
        sk0 = own && h0 + n16 < a.H ? ssink[hb * 32 + n16] * kLog2e : -INFINITY;
        sk1 = own && h0 + 16 + n16 < a.H ? ssink[hb * 32 + 16 + n16] * kLog2e : -INFINITY;
      }
      const int ntiles = (n + kSuper - 1) / kSuper;

      auto issue_tile = [&](int tile) { issue_super(n, tile); };
      const int first_burst = ntiles < kBurst ? ntiles : kBurst;
      if (sc > 0 || pass > 0)  // the first chunk's burst went out in the prologue
        for (int k = 0; k < first_burst; ++k) issue_tile(k);

      for (int i = 0; i < ntiles; ++i) {
        // before this wait, tiles [0, first_burst) went out together and one
        // more after each barrier from i = 1 on: min(ntiles, kBurst + i - 1)
        const int issued = i == 0 ? first_burst : min(ntiles, kBurst + i - 1);
        wait_outstanding(issued - i - 1);
        barrier_lds();  // super-tile i is in LDS; every wave is done with i-1's stage
        // the next tile goes into the stage tile i - 1 left (kBurst <= kStages)
        if (i >= 1 && i - 1 + kBurst < ntiles) issue_tile(i - 1 + kBurst);

        const int nvalid = n - i * kSuper - 16 * par;  // rows of this wave's 16 that exist
        if (nvalid <= 0) continue;                     // (wave-uniform: a ragged tail)
        // The stage's offset is opaque to the compiler: it would otherwise keep
        // every lane offset precomputed for each stage (registers it lacks).
        int stoff = (i % kStages) * kStageBytes + 16 * par * kRowBytes;
        asm volatile("" : "+v"(stoff));
        const unsigned char* st = smem + stoff;

        if constexpr (kFp8) {
          // S^T = K Q^T for both head blocks over codes: per k-step the code
          // read of step u + kKA, the exact decode of step u and its two
          // MFMAs (a fence per step keeps kKA + 1 steps of codes live)
          u32x2 ra[kKSteps];
          f32x4 s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
#pragma unroll
          for (int u = 0; u < kKA && u < kKSteps; ++u) ra[u] = *reinterpret_cast<const u32x2*>(st + off8.kq(u));
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            if (u + kKA < kKSteps) ra[u + kKA] = *reinterpret_cast<const u32x2*>(st + off8.kq(u + kKA));
            const bf16x8 ka = e4m3x8_to_bf16(ra[u]);
            if (u & 1) {
              s0b = mfma_k32(ka, q0[u], s0b);
              s1b = mfma_k32(ka, q1[u], s1b);
            } else {
              s0a = mfma_k32(ka, q0[u], s0a);
              s1a = mfma_k32(ka, q1[u], s1a);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          const f32x4 s0 = s0a + s0b, s1 = s1a + s1b;

          // the scales of this lane's rows 16 par + 4 g .. + 3 (row r of the
          // super-tile was loaded by wave r / kRowsPerWave into its entry
          // r % kRowsPerWave); they multiply the scores, and the weights
          // before these are rounded to bf16
          const int r0 = 16 * par + 4 * g;
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(
              &sscale[i % (kFp8 ? kStages : 1)][r0 / kRowsPerWave][r0 % kRowsPerWave]);
          float x0[4], x1[4];
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const bool v = 4 * g + i4 < nvalid;
            x0[i4] = v ? s0[i4] * (a.qk_scale * c0[i4]) : -INFINITY;
            x1[i4] = v ? s1[i4] * (a.qk_scale * c0[i4]) : -INFINITY;
          }
          float pf0[4], pf1[4];
          over |= softmax_tile_f32<4>(x0, sk0, g, first0, m0, mt0, l0, pf0);
          over |= softmax_tile_f32<4>(x1, sk1, g, first1, m1, mt1, l1, pf1);
          bf16x4 pa, pbk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pa[e] = (__bf16)(pf0[e] * c0[e]);
            pbk[e] = (__bf16)(pf1[e] * c0[e]);
          }
          const bf16x8 pb = wide_p_operand(pa, pbk);

          // O^T += V^T P^T over the 16 rows: the 8-bit transposing read of
          // d-tile u + kVA, the decode of d-tile u and its MFMA
          u32x2 va[kDT];
          auto read_vt = [&](int u) {
            va[u] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsV2i32*)(st + voff8.at(u))));
          };
#pragma unroll
          for (int u = 0; u < kVA && u < kDT; ++u) read_vt(u);
#pragma unroll
          for (int u = 0; u < kDT; ++u) {
            if (u + kVA < kDT) read_vt(u + kVA);
            acc[u] = mfma32(e4m3x8_to_bf16(va[u]), pb, acc[u]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          // S^T = K Q^T for both head blocks; the K reads run kKA k-steps ahead
          // of the MFMAs that consume them (one read issued after each step's
          // MFMA pair), two chains per block.
          bf16x8 ka[kKSteps];
          f32x4 s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
#pragma unroll
          for (int u = 0; u < kKA && u < kKSteps; ++u) ka[u] = *reinterpret_cast<const bf16x8*>(st + off.kq(u));
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            if (u & 1) {
              s0b = mfma_k32(ka[u], q0[u], s0b);
              s1b = mfma_k32(ka[u], q1[u], s1b);
            } else {
              s0a = mfma_k32(ka[u], q0[u], s0a);
              s1a = mfma_k32(ka[u], q1[u], s1a);
            }
            if (u + kKA < kKSteps) ka[u + kKA] = *reinterpret_cast<const bf16x8*>(st + off.kq(u + kKA));
          }
          {
            constexpr int kPre = kKA < kKSteps ? kKA : kKSteps;
            __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
            for (int u = 0; u < kKSteps; ++u) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              if (u + kPre < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          const f32x4 s0 = s0a + s0b, s1 = s1a + s1b;

          float x0[4], x1[4];
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const bool v = 4 * g + i4 < nvalid;
            x0[i4] = v ? s0[i4] * a.qk_scale : -INFINITY;
            x1[i4] = v ? s1[i4] * a.qk_scale : -INFINITY;
          }
          __bf16 p0[4], p1[4];
          over |= softmax_tile<4>(x0, sk0, g, first0, m0, mt0, l0, p0);
          over |= softmax_tile<4>(x1, sk1, g, first1, m1, mt1, l1, p1);
          bf16x4 pa, pbk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pa[e] = p0[e];
            pbk[e] = p1[e];
          }
          const bf16x8 pb = wide_p_operand(pa, pbk);

          // O^T += V^T P^T over the 16 rows: the two transposing reads of d-tile
          // u + kVA run under the MFMA of d-tile u.
          {
            bf16x8 va[kDT];
            auto read_vt = [&](int u) {
              const bf16x4 vl = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + voff.at(u, 0)));
              const bf16x4 vh = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + voff.at(u, 1)));
              va[u] = __builtin_shufflevector(vl, vh, 0, 1, 2, 3, 4, 5, 6, 7);
            };
#pragma unroll
            for (int u = 0; u < kVA && u < kDT; ++u) read_vt(u);
#pragma unroll
            for (int u = 0; u < kDT; ++u) {
              acc[u] = mfma32(va[u], pb, acc[u]);
              if (u + kVA < kDT) read_vt(u + kVA);
            }
            constexpr int kPre = kVA < kDT ? kVA : kDT;
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);
#pragma unroll
            for (int u = 0; u < kDT; ++u) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              if (u + kPre < kDT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    if (!workgroup_any(over, sflag, wave, kWaves)) break;
  }

  // This wave's states: head n16 of block 0 (m0, l0) and of block 1 (m1, l1);
  // m is -inf for a parity that saw no row.  Accumulator layout: lane
  // (n = lane % 32, hf = lane / 32) holds, for head h0 + n, d = out_col(dt,
  // e4) + 4 hf + e as element 4 e4 + e of acc[dt]; head h0 + n is head n % 16 =
  // lane % 16 of block n / 16, whose softmax state this lane holds too.
  const int n = lane & 31, hf = lane >> 5;
  // bf16 rows: the columns in order; FP8 rows: the 16-column chunks in the
  // order of the transposing reads (wide_vt_chunk)
  auto out_col = [](int dt, int e4) {
    if constexpr (kFp8)
      return 16 * wide_vt_chunk<D>(dt, e4 >> 1) + 8 * (e4 & 1);
    else
      return 32 * dt + 8 * e4;
  };
  float lb0 = group_sum4(l0), lb1 = group_sum4(l1);

  // Merge the P parity states of head block hb in LDS: a butterfly over the
  // parity bits.  At stride s a wave keeps the lower half of its current
  // d-tile range when bit s of its parity is 0 (the upper one otherwise),
  // hands the other half to its partner par ^ s, and combines the partner's
  // half with its own, the lower parity's state first.
  int lo = 0;  // first d-tile of the range this wave holds; acc[0, kDTw) is the piece
  if constexpr (P > 1) {
#pragma unroll
    for (int s = 1; s < P; s <<= 1) {
      constexpr int kHalfMax = kDT / 2;
      const int half = kDT / (2 * s);  // compile-time per unrolled round
      const bool upper = (par & s) != 0;
      const int partner = hb * P + (par ^ s);
      barrier_lds();  // the ring is free, and the previous round's reads are done
      if (g == 0) {
        sml[wave][0][n16] = m0;
        sml[wave][1][n16] = m1;
        sml[wave][2][n16] = lb0;
        sml[wave][3][n16] = lb1;
      }
      // hand over the half this wave gives away (register image); the
      // branches are wave-uniform and keep every accumulator index constant
      f32x4* mine = reinterpret_cast<f32x4*>(smem) + wave * kHalfMax * 256 + lane;
      if (upper) {
#pragma unroll
        for (int i = 0; i < half; ++i)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) mine[(i * 4 + e4) * 64] = quarter(acc[i], e4);
      } else {
#pragma unroll
        for (int i = 0; i < half; ++i)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) mine[(i * 4 + e4) * 64] = quarter(acc[half + i], e4);
      }
      barrier_lds();
      const float pm0 = sml[partner][0][n16], pm1 = sml[partner][1][n16];
      const float pl0 = sml[partner][2][n16], pl1 = sml[partner][3][n16];
      const float M0 = fmaxf(m0, pm0), M1 = fmaxf(m1, pm1);
      const float ws0 = state_weight(m0, M0), wp0 = state_weight(pm0, M0);
      const float ws1 = state_weight(m1, M1), wp1 = state_weight(pm1, M1);
      const float wself = n < 16 ? ws0 : ws1, wpart = n < 16 ? wp0 : wp1;
      const f32x4* tp = reinterpret_cast<const f32x4*>(smem) + partner * kHalfMax * 256 + lane;
      // the kept half moves to the front, the lower parity's state first
      if (upper) {
#pragma unroll
        for (int i = 0; i < half; ++i) {
          f32x16 other;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) set_quarter(other, e4, tp[(i * 4 + e4) * 64]);
          acc[i] = wpart * other + wself * acc[half + i];
        }
        lb0 = wp0 * pl0 + ws0 * lb0;
        lb1 = wp1 * pl1 + ws1 * lb1;
        lo += half;
      } else {
#pragma unroll
        for (int i = 0; i < half; ++i) {
          f32x16 other;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) set_quarter(other, e4, tp[(i * 4 + e4) * 64]);
          acc[i] = wself * acc[i] + wpart * other;
        }
        lb0 = ws0 * lb0 + wp0 * pl0;
        lb1 = ws1 * lb1 + wp1 * pl1;
      }
      m0 = M0;
      m1 = M1;
    }
  }

  // Cross-workgroup merge, a reduce-scatter.  Piece w (held by wave w: head
  // block w / P, d-tiles [piece_lo(w % P), + kDTw)) is cut into U units of
  // du = kDTw / U d-tiles, U the least power of two with 4 U >= nparts (at
  // most kDTw), and unit u = w U + j is merged by partition u mod nparts: the
  // merge reads spread over up to 4 U workgroups instead of four.  Every
  // partition publishes its pieces and counts itself in on each unit another
  // partition merges; a merging workgroup waits for its unit's count
  // (bounded), then each of its waves sums a quarter of the unit's columns
  // over every partition's share, in partition order.
  auto piece_lo = [](int pr) {  // first d-tile a parity keeps after the butterfly
    int l = 0;
#pragma unroll
    for (int s2 = 1; s2 < P; s2 <<= 1) l += (pr & s2) ? kDT / (2 * s2) : 0;
    return l;
  };
  if (nparts == 1) {
    // out = O / l for heads h0 + n, d-tiles [lo, lo + kDTw)
    if (h0 + n < a.H) {
      const float inv = 1.0f / (n < 16 ? lb0 : lb1);
      uint16_t* op = a.out + ((int64_t)t * a.H + h0 + n) * D + 4 * hf;
#pragma unroll
      for (int i = 0; i < kDTw; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) store_bf16x4(op + out_col(lo + i, e4), quarter(acc[i], e4), inv);
    }
    return;
  }

  const int64_t slot = (int64_t)Pc::kBytes;
  const int64_t item_bytes = kWaves * slot;
  unsigned char* ws = reinterpret_cast<unsigned char*>(a.ws);
  // the slot of the (token, head group)'s partition 0 (its partitions' slots
  // follow it), and the number of slots, behind which the counters start
  int64_t slot0, n_items;
  if (a.bal_slots > 0) {
    const int j = xcd_item(blockIdx.x, gridDim.x) - hg * a.bal_slots;
    slot0 = (int64_t)hg * a.bal_slots + (j - c);
    n_items = (int64_t)a.head_groups * a.bal_slots;
  } else {
    slot0 = (int64_t)th * a.splits;
    n_items = (int64_t)a.N * a.head_groups * a.splits;
  }
  unsigned char* ws_th = ws + slot0 * item_bytes;
  // kDTw arrival counters a piece (one a unit at the finest cut)
  int* ctr_th = reinterpret_cast<int*>(ws + n_items * item_bytes) + (int64_t)th * kWaves * kDTw;
  const int others = nparts - 1;
  int U = 1;
  while (U < kDTw && 4 * U < nparts) U <<= 1;
  const int du = kDTw / U;
  auto ctr_of = [&](int u) { return ctr_th + (u / U) * kDTw + u % U; };

  // publishing: this wave's piece to its slot, complete before any count
  auto publish = [&]() {
    const __amdgpu_buffer_rsrc_t r = ws_rsrc(ws_th + c * item_bytes + wave * slot);
#pragma unroll
    for (int i = 0; i < kDTw; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) store_bf16x4_sc1(r, ((i * 4 + e4) * 64 + lane) * 8, quarter(acc[i], e4));
    if (g == 0) {
      store1_sc1(r, Pc::kOBytes + n16 * 4, m0);
      store1_sc1(r, Pc::kOBytes + (16 + n16) * 4, m1);
      store1_sc1(r, Pc::kOBytes + 128 + n16 * 4, lb0);
      store1_sc1(r, Pc::kOBytes + 128 + (16 + n16) * 4, lb1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // Merge of quarter-columns [v kQ, (v + 1) kQ) of unit u (kQ = du) by one
  // wave: every partition's share of them, this one's included, from the
  // slots, summed in partition order with a running maximum (so every arrival
  // order gives the same bits).  Writes out.
  auto merge_part = [&](int u, int v, auto q_tag) {
    constexpr int kQ = decltype(q_tag)::value;
    // partitions whose shares are loaded together
    constexpr int kB = kQ == 1 ? 16 : (kQ == 2 ? 8 : 32 / kQ);
    const int w = u / U;
    const int i0 = (u % U) * du;  // the unit's first d-tile within the piece
    float M0 = -INFINITY, M1 = -INFINITY, ls0 = 0.f, ls1 = 0.f;
    f32x4 tot[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) tot[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one descriptor over the (token, head group)'s slots; a partition's slot
    // is a scalar offset from it (< 2^31: at most 32 partitions of 4 slots)
    const __amdgpu_buffer_rsrc_t r = ws_rsrc(ws_th);
    for (int k0 = 0; k0 < nparts; k0 += kB) {
      f32x4 x[kB][kQ];
      float bm0[kB], bm1[kB], bl0[kB], bl1[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) {  // the batch's loads go out before any is used
        const int k = k0 + b < nparts ? k0 + b : k0;  // (past nparts: a repeat, unused)
        const int so = __builtin_amdgcn_readfirstlane((int)(k * item_bytes + w * slot));
        bm0[b] = load1_sc1(r, Pc::kOBytes + n16 * 4, so);
        bm1[b] = load1_sc1(r, Pc::kOBytes + (16 + n16) * 4, so);
        bl0[b] = load1_sc1(r, Pc::kOBytes + 128 + n16 * 4, so);
        bl1[b] = load1_sc1(r, Pc::kOBytes + 128 + (16 + n16) * 4, so);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const int qc = v * kQ + q;
          x[b][q] = load_bf16x4_sc1(r, (((i0 + qc / 4) * 4 + qc % 4) * 64 + lane) * 8, so);
        }
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (k0 + b < nparts) {
          const float N0 = fmaxf(M0, bm0[b]), N1 = fmaxf(M1, bm1[b]);
          const float s0 = state_weight(M0, N0), s1 = state_weight(M1, N1);
          const float w0 = state_weight(bm0[b], N0), w1 = state_weight(bm1[b], N1);
          ls0 = s0 * ls0 + w0 * bl0[b];
          ls1 = s1 * ls1 + w1 * bl1[b];
          const float sk = n < 16 ? s0 : s1, wk = n < 16 ? w0 : w1;
#pragma unroll
          for (int q = 0; q < kQ; ++q) tot[q] = sk * tot[q] + wk * x[b][q];
          M0 = N0;
          M1 = N1;
        }
      }
    }
    const int hw0 = hg * kHeads + (w / P) * 32;  // first head of piece w
    if (hw0 + n < a.H) {
      const float inv = 1.0f / (n < 16 ? ls0 : ls1);
      uint16_t* op = a.out + ((int64_t)t * a.H + hw0 + n) * D + 4 * hf;
      const int dt0 = piece_lo(w % P) + i0;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int qc = v * kQ + q;
        store_bf16x4(op + out_col(dt0 + qc / 4, qc % 4), tot[q], inv);
      }
    }
  };
  auto merge_unit_part = [&](int u, int v) {  // du: a power of two, at most kDTw
    if (du == 1) {
      merge_part(u, v, std::integral_constant<int, 1>{});
    } else if (du == 2) {
      if constexpr (kDTw >= 2) merge_part(u, v, std::integral_constant<int, 2>{});
    } else if (du == 4) {
      if constexpr (kDTw >= 4) merge_part(u, v, std::integral_constant<int, 4>{});
    } else {
      if constexpr (kDTw >= 8) merge_part(u, v, std::integral_constant<int, 8>{});
    }
  };

  // 1. every wave publishes its piece, then counts itself in on each unit of
  //    it that another partition merges (lane j on unit j, all at once); an
  //    arrival that completes a count whose merger gave up merges that unit
  //    alone
  publish();
  {
    const int u = wave * U + lane;
    int old = -1;
    if (lane < U && u % nparts != c)
      old = __hip_atomic_fetch_add(ctr_of(u), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t done = __builtin_amdgcn_ballot_w64(old == others);
    asm volatile("" ::: "memory");
    while (done != 0) {  // (wave-uniform)
      const int uj = wave * U + __builtin_ctzll(done);
      done &= done - 1;
      // one wave takes all 4 du quarter-columns, at most four a call (wider
      // calls here would hold more registers than the kernel has)
      if (du >= 4) {
        if constexpr (kDTw >= 4)
          for (int v = 0; v < du; ++v) merge_part(uj, v, std::integral_constant<int, 4>{});
      } else if (du == 2) {
        if constexpr (kDTw >= 2)
          for (int v = 0; v < 4; ++v) merge_part(uj, v, std::integral_constant<int, 2>{});
      } else {
        for (int v = 0; v < 4; ++v) merge_part(uj, v, std::integral_constant<int, 1>{});
      }
      if (lane == 0) __hip_atomic_store(ctr_of(uj), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // 2. the units this workgroup merges (u = c, c + nparts, ...), its four
  //    waves sharing the columns of each
  int* sdec = sflag;
  for (int u = c; u < kWaves * U; u += nparts) {  // (workgroup-uniform)
    barrier_lds();  // every wave has read the previous unit's decision
    if (wave == 0) {  // wait for the other partitions' counts
      int* cu = ctr_of(u);
      int v = 0;
      const uint64_t t_spin = __builtin_amdgcn_s_memrealtime();
      const uint64_t extra = short_rows > 0 ? (uint64_t)short_rows * kSpinTicksPerRow : 0;
      const uint64_t spin_ticks =
          kSpinTicks + extra < kSpinTicksMax ? kSpinTicks + extra : kSpinTicksMax;
      for (int it = 0; a.split_wait && it < kSpinLimit; ++it) {
        // polled with a read-modify-write (max with 0 leaves the count as it
        // is): it is served where the arrivals' adds are, which a plain
        // agent-scope load is not guaranteed to be promptly
        if (lane == 0) v = __hip_atomic_fetch_max(cu, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = __builtin_amdgcn_readfirstlane(v);
        if (v >= others) break;
        if (__builtin_amdgcn_s_memrealtime() - t_spin > spin_ticks) break;
        __builtin_amdgcn_s_sleep(2);
      }
      asm volatile("" ::: "memory");
      int decision = 1;
      if (v < others) {  // (waited long enough, or not at all) the arrival that completes the count merges
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(cu, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        decision = __builtin_amdgcn_readfirstlane(old) == others ? 1 : 0;
        asm volatile("" ::: "memory");
      }
      if (decision && lane == 0) __hip_atomic_store(cu, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) sdec[0] = decision;
    }
    barrier_lds();
    if (sdec[0] == 0) continue;  // (workgroup-uniform) a later arrival merges it
    merge_unit_part(u, wave);
  }
}

// Compute units of the current device, read once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int HB, int P, bool kFp8>
hipError_t launch_split_d(const AttnArgs& a0, const AttnPlan& p, hipStream_t stream) {
  const long long items = p.bal_slots > 0 ? (long long)a0.head_groups * p.bal_slots
                                          : (long long)a0.N * a0.head_groups * a0.splits;
  AttnArgs a = a0;
  a.bal_slots = p.bal_slots;
  // one workgroup per CU (the LDS ring and 512 registers a wave): the grid is
  // resident at once when it has no more workgroups than CUs
  a.split_wait = items <= device_cus() ? 1 : 0;
  hipLaunchKernelGGL((attn_split_kernel<D, HB, P, kFp8>), dim3((unsigned)items), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool kFp8>
hipError_t launch_split_shape(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  const int hb = p.heads_per_group / 32;
  if (hb == 2 && p.parities == 2) return launch_split_d<D, 2, 2, kFp8>(a, p, stream);
  if constexpr (D >= 128) {
    if (hb == 1 && p.parities == 4) return launch_split_d<D, 1, 4, kFp8>(a, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t split_counters_offset(int32_t N, int32_t D, const AttnPlan& p) {
  const size_t slot = (size_t)(D / 32 / p.parities) * 4 * 64 * 8 + 2 * 32 * 4;
  const size_t items = p.bal_slots > 0 ? (size_t)p.head_groups * p.bal_slots
                                        : (size_t)N * p.head_groups * p.splits;
  return items * 4 * slot;
}

size_t split_workspace_bytes(int32_t N, int32_t D, const AttnPlan& p) {
  // one arrival counter per unit at the finest cut: D / 32 / parities a piece
  return split_counters_offset(N, D, p) +
         (size_t)N * p.head_groups * 4 * (D / 32 / p.parities) * sizeof(int);
}

hipError_t launch_split(const AttnArgs& a, int D, const AttnPlan& p, bool fp8, hipStream_t stream) {
  if (fp8) {
    switch (D) {
      case 128: return launch_split_shape<128, true>(a, p, stream);
      case 256: return launch_split_shape<256, true>(a, p, stream);
      case 512: return launch_split_shape<512, true>(a, p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (D) {
    case 64: return launch_split_shape<64, false>(a, p, stream);
    case 128: return launch_split_shape<128, false>(a, p, stream);
    case 256: return launch_split_shape<256, false>(a, p, stream);
    case 512: return launch_split_shape<512, false>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spd
