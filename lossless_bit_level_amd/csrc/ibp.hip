// libibp: Invariant Bit Packing for AMD Instinct MI355X (gfx950, CDNA4).
//
// Method source, cited as [IBP]: the explainer page "Reducing the GPU Memory
// Bottleneck with Lossless Compression for ML -- Extended" (Kamath,
// Krishnamurthy, Canini, Peter), section "Methodology: Invariant Bit Packing
// (IBP)" (phases Preprocessing, Compression, Decompression) and section
// "System integration" (fixed-size buffers, GPU bitmask of compressed rows).
// The image format is specified in include/ibp.h.
//
// Everything here is integer bit work bound by HBM (or by the host link for a
// pinned image); nothing is a contraction, so no MFMA.  Design for wave64:
//   * a 64-block chunk of a row maps to one wave, one block per lane;
//   * the participation bits of the chunk are one 64-bit header word, so the
//     offset of each lane's payload is a closed-form prefix count:
//     v_mbcnt_lo/hi over the header word plus a scalar carry (s_bcnt1) --
//     the wave prefix scan of the per-block bit lengths, which take only the
//     two values 1 + W - p and 1 + W;
//   * the compressed stream of a row segment is fetched by the wave with
//     coalesced 16-byte loads into a wave-private LDS window, and each lane
//     pulls its payload out of two LDS words with one funnel shift;
//   * invariant bits go back in with a run decomposition of ~Mask
//     (v_bfe_u32 + v_lshl_or_b32 per run) and an OR with Bitval; the run
//     count is a template parameter for the common masks;
//   * workgroups keep the dispatcher's order (round robin over the 8 XCDs):
//     renumbering them so that consecutive tasks share an XCD and its L2
//     made every decode from HBM slower, by 4-11%; only segment decodes from
//     a host image renumber (xcd_remap).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "ibp.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / kWave;
constexpr uint32_t kSegBlocks = 1024;          // blocks per decode task
constexpr uint32_t kSegLdsWords = kSegBlocks + 8;
constexpr uint64_t kMaxRowBytes = 1ull << 26;  // bit offsets fit 32 bits, counts 24
constexpr int kMaxRuns = 16;                   // runs of ~Mask for W = 32
constexpr uint32_t kMaxGrid = 1u << 24;
constexpr uint32_t kSpecWords = 32;            // first slot words fetched with the header
constexpr uint32_t kSlotPipeMaxP = 8;          // row pipelines fetch whole slots up to this p

// Run decomposition of the kept (non-invariant) bit positions ~Mask.  Run j
// is a maximal stretch of kept block bits; `place[j]` is its mask in the
// block, `shift[j]` how far it moves between block and payload (its block
// position minus the number of kept bits below it, always >= 0).  Then
//   extract:  payload = OR_j ((x & place[j]) >> shift[j])
//   deposit:  block   = OR_j ((v << shift[j]) & place[j])
// two VALU ops per run either way.
struct Runs {
  uint32_t n;
  uint32_t shift[kMaxRuns];
  uint32_t place[kMaxRuns];
};

struct Codec {
  uint32_t mask;
  uint32_t bitval;
  uint32_t p;       // invariant bits
  uint32_t n;       // blocks per row
  uint32_t pad;     // compression: stored rows padded to 64-byte units (device slots)
  Runs runs;
};

// Parallel bit extract by ~Mask: [IBP] Compression strips the invariant bits
// and closes the gaps.
template <int NR>
__device__ __forceinline__ uint32_t extract_kept(uint32_t x, const Runs& rs) {
  uint32_t v = 0;
  if constexpr (NR >= 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) v |= (x & rs.place[j]) >> rs.shift[j];
  } else {
    for (uint32_t j = 0; j < rs.n; ++j) v |= (x & rs.place[j]) >> rs.shift[j];
  }
  return v;
}

// Parallel bit deposit by ~Mask, ORed onto `base`: [IBP] Decompression puts
// the stored bits back around the invariant positions (base = Bitval).
template <int NR>
__device__ __forceinline__ uint32_t deposit_kept(uint32_t v, const Runs& rs, uint32_t base) {
  uint32_t x = base;
  if constexpr (NR >= 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) x |= (v << rs.shift[j]) & rs.place[j];
  } else {
    for (uint32_t j = 0; j < rs.n; ++j) x |= (v << rs.shift[j]) & rs.place[j];
  }
  return x;
}

__device__ __forceinline__ uint32_t lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// v_writelane_b32: `old` with lane `lane` (a constant) set to the scalar v
// (the intrinsic, which this compiler has no builtin for).
__device__ int lane_write(int v, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// v_mul_i32_i24: the product of the low 24 bits of a and b, as signed values.
__device__ int mul_i24(int a, int b) __asm("llvm.amdgcn.mul.i24.i32");

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Number of set bits of the 64-bit word (hi:lo) strictly below this lane.
__device__ __forceinline__ uint32_t bits_below_lane(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
}

// The same plus acc (v_mbcnt accumulates into its second operand).
__device__ __forceinline__ uint32_t bits_below_lane_acc(uint32_t lo, uint32_t hi, uint32_t acc) {
  return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, acc));
}

// Sum over the 64 lanes with DPP row shifts and row broadcasts (an inclusive
// scan; lane 63 ends up with the total), result in a scalar register.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, uint32_t lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t t = __shfl_up(v, d, kWave);
    if (lane >= (uint32_t)d) v += t;
  }
  return v;
}

// Make this wave's LDS writes visible to its own later LDS reads (one wave
// executes its LDS instructions in order; this stops compiler reordering).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Buffer resource over `bytes` bytes at p (gfx9 word 3: 32-bit data format).
// A buffer load past `bytes` returns zeros and moves no data, and a store
// past it is dropped, so an access whose lanes partly or wholly fall outside
// a row's stream needs no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache policy (aux operand) of a buffer load of the part of a stream past
// its first 128 bytes: non-temporal, as stage_window's loads.
constexpr int kLoadStream = 2;

// Cache policy of the compressors' row loads and stores: non-temporal (a raw
// row is read once and a stored row written once).
constexpr int kRowLoad = 2;
constexpr int kRowStore = 2;

// Words to write for a compressed row whose stream has `words` words, at slot
// address row (slots of n words): with pad (device memory), on to the next
// 64-byte boundary of the address, at most n.  A write that ends inside a
// 64-byte unit costs HBM a read-modify-write: copying 2 GiB of 512-byte rows
// took 0.98 ms writing 464 bytes of each and 0.78 ms writing all 512.  The
// added words are zeros.
__device__ __forceinline__ uint32_t store_words(const void* row, uint32_t words, uint32_t n,
                                                uint32_t pad) {
  if (!pad) return words;
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(row) >> 2) & 15u;
  return min(n, ((a + words + 15u) & ~15u) - a);
}

// 16 bytes as a native vector (kept in registers; HIP's uint4 struct is not
// always promoted out of private memory when it is assigned conditionally).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Copy units [0, cnt) of g into the wave's LDS window l (16-byte units when
// U is u32x4, words when U is uint32_t).  All loads of a batch of MAXV units
// per lane are issued before the first LDS write, so that a window costs one
// memory latency per batch, not one per 64 units (a plain strided loop waits
// for each load before its LDS write).  With NT the loads are non-temporal.
// Measured on MI355X: for the bulk of a stream, past the 128-byte window a
// row's first load takes, that is faster (a weight layer 1% and KV pages
// 5.5% faster; per-position KV pages 5.5% with the row pipeline's loads of
// the same part); for the windows themselves, short scattered reads, and
// for whole short slots read again and again (Zipf ids) it is much slower,
// so those keep the default policy, as does the cache arena, whose rows are
// read again.  cnt is wave-uniform.
template <int MAXV, bool NT = false, typename U>
__device__ __forceinline__ void stage_window(const U* __restrict__ g, U* l, uint32_t cnt,
                                             uint32_t lane) {
  for (uint32_t j0 = 0; j0 < cnt; j0 += MAXV * kWave) {
    U v[MAXV];
#pragma unroll
    for (int c = 0; c < MAXV; ++c) {
      const uint32_t j = j0 + c * kWave + lane;
      if constexpr (NT)
        v[c] = j < cnt ? __builtin_nontemporal_load(g + j) : U{};
      else
        v[c] = j < cnt ? g[j] : U{};
    }
#pragma unroll
    for (int c = 0; c < MAXV; ++c) {
      const uint32_t j = j0 + c * kWave + lane;
      if (j < cnt) l[j] = v[c];
    }
  }
}

// One block per lane: pull the payload at bit `rel` of the LDS window out of
// two words with a funnel shift; a stripped block (its bit set in the 64-bit
// chunk header, used directly as a lane mask) gets its invariant bits back.
__device__ __forceinline__ uint32_t lds_bits(const uint32_t* lds, uint32_t rel) {
  const uint32_t wi = __builtin_amdgcn_ubfe(rel, 5, 27);
  return __builtin_amdgcn_alignbit(lds[wi + 1], lds[wi], rel & 31u);
}

// Workgroups are handed to the 8 XCDs round robin; this renumbering gives
// each XCD a contiguous range of logical workgroups (a bijection on [0, G)).
// Only decodes from a host image use it: there the segments of one row then
// read their shared header words across the host link once per XCD L2, not
// once per segment.  From HBM the dispatcher's order is faster.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t g) {
  const uint32_t x = 8;
  uint32_t q = g / x, r = g % x, xcd = b % x, idx = b / x;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// v_bitop3 with truth table 0xE4 is a bitwise select, S2 ? S0 : S1 (one
// instruction, whether the mask sits in a vector or a scalar register).
__device__ __forceinline__ uint32_t select_bits(uint32_t mask, uint32_t a, uint32_t b) {
  return __builtin_amdgcn_bitop3_b32(a, b, mask, 0xE4);
}

template <int NR>
__device__ __forceinline__ uint32_t decode_block(const uint32_t* lds, uint32_t rel,
                                                 uint32_t h_lo, uint32_t h_hi,
                                                 const Codec& cd) {
  const uint32_t v = lds_bits(lds, rel);
  const uint32_t dep = deposit_kept<NR>(v, cd.runs, cd.bitval);
  const bool stripped =
      __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
  return stripped ? dep : v;
}

// ------------------------------------------------------------ kernels --

// Where a decode task finds its row.
constexpr int kModeTable = 0;   // row i of the image (full decompress)
constexpr int kModeGather = 1;  // row ids[i] of the image
constexpr int kModeCached = 2;  // row ids[i]: the packed cache entry when resident, else the image

// First word of a row: its cache entry (locator resident), else its slot.
template <int MODE>
__device__ __forceinline__ const uint32_t* row_source(const uint32_t* slots,
                                                      const uint32_t* arena, uint64_t id,
                                                      uint32_t n, unsigned long long loc) {
  if constexpr (MODE == kModeCached)
    if (loc & IBP_LOC_RESIDENT) return arena + (loc & IBP_LOC_OFFSET_MASK) * 4;
  return slots + id * n;
}

// Words that may be read from there: the entry's stored words, or the slot.
template <int MODE>
__device__ __forceinline__ uint32_t row_words(uint32_t n, unsigned long long loc) {
  if constexpr (MODE == kModeCached)
    if (loc & IBP_LOC_RESIDENT) return (uint32_t)((loc >> IBP_LOC_WORDS_SHIFT) & IBP_LOC_WORDS_MASK);
  return n;
}

// Stored compressed?  From the locator of a cached row, else the image's
// flag word fw (the word holding bit id & 63).
template <int MODE>
__device__ __forceinline__ bool row_flag(unsigned long long fw, uint64_t id,
                                         unsigned long long loc) {
  if constexpr (MODE == kModeCached)
    if (loc & IBP_LOC_RESIDENT) return (loc & IBP_LOC_COMPRESSED) != 0;
  return (fw >> (id & 63)) & 1ull;
}



__global__ void fill_u64_kernel(unsigned long long* p, uint64_t n, unsigned long long v) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// [IBP] Preprocessing, device half: per-bit one counts over the sample.
//
// Bit-sliced counting.  A lane takes 32 blocks per step (eight 16-byte loads,
// each coalesced over the wave) and adds them with a tree of ripple-carry
// adders that works on all 32 bit positions at once: afterwards bit b of
// plane j is bit j of the number of ones at position b among those blocks.
// That 6-plane number is added into a P-plane accumulator the same way, and
// only after the last step are the planes turned into 32 counters and summed
// over the wave.  About 7 VALU per block and no scalar work in the loop; a
// ballot per bit would cost 32 ballots plus their scalar popcounts per block,
// on a scalar unit that the four SIMDs of a CU share.
constexpr int kCountWords = 32;                              // blocks per lane per step
constexpr uint32_t kCountGroup = kCountWords * kWave;        // words per wave step
constexpr uint64_t kCountMaxSteps = (1u << 24) / kCountWords - 1;  // per wave, so P <= 24

// out[0..B] = x[0..B) + y[0..B), bit-sliced.
template <int B>
__device__ __forceinline__ void sliced_add(const uint32_t* x, const uint32_t* y, uint32_t* out) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < B; ++j) {
    const uint32_t t = x[j] ^ y[j];
    out[j] = t ^ c;
    c = (x[j] & y[j]) | (c & t);
  }
  out[B] = c;
}

// acc += s, bit-sliced; the caller keeps every position's total below 2^P.
template <int P, int S>
__device__ __forceinline__ void sliced_accumulate(uint32_t (&acc)[P], const uint32_t (&s)[S]) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const uint32_t a = acc[j];
    if (j < S) {
      const uint32_t t = a ^ s[j];
      acc[j] = t ^ c;
      c = (a & s[j]) | (c & t);
    } else {
      acc[j] = a ^ c;
      c = a & c;
    }
  }
}

// Ones per position among the 32 blocks w[], as 6 planes.
__device__ __forceinline__ void sliced_count32(const uint32_t (&w)[kCountWords], uint32_t (&s)[6]) {
  uint32_t l1[16][2], l2[8][3], l3[4][4], l4[2][5];
#pragma unroll
  for (int i = 0; i < 16; ++i) sliced_add<1>(&w[2 * i], &w[2 * i + 1], l1[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) sliced_add<2>(l1[2 * i], l1[2 * i + 1], l2[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) sliced_add<3>(l2[2 * i], l2[2 * i + 1], l3[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) sliced_add<4>(l3[2 * i], l3[2 * i + 1], l4[i]);
  sliced_add<5>(l4[0], l4[1], s);
}

// The same for 16 blocks, as 5 planes.
__device__ __forceinline__ void sliced_count16(const uint32_t (&w)[16], uint32_t (&s)[5]) {
  uint32_t l1[8][2], l2[4][3], l3[2][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) sliced_add<1>(&w[2 * i], &w[2 * i + 1], l1[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) sliced_add<2>(l1[2 * i], l1[2 * i + 1], l2[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) sliced_add<3>(l2[2 * i], l2[2 * i + 1], l3[i]);
  sliced_add<4>(l3[0], l3[1], s);
}

// Step g of the sample covers words [g*2048, (g+1)*2048): lane L takes the
// four words of 16-byte unit g*512 + j*64 + L for j < 8.  Words past the
// end read as 0 (they add no ones).  NPOS = 32 counts the 32 bit positions
// of every word; NPOS = 64 counts even and odd words apart (the low and high
// halves of 64-bit blocks: a word's parity is that of its component in the
// unit).  Partial counts go out transposed, partials[b * gridDim.x +
// workgroup], so the reduction reads each position's column contiguously.
template <int P, int NPOS>
__global__ __launch_bounds__(kBlockThreads) void count_ones_kernel(
    const uint32_t* __restrict__ sample, uint64_t n_blocks,
    unsigned long long* __restrict__ partials) {
  static_assert(NPOS == 32 || NPOS == 64, "32 or 64 positions");
  constexpr int NACC = NPOS / 32;
  __shared__ uint32_t part[kWavesPerBlock][NPOS];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint64_t gwave = (uint64_t)blockIdx.x * kWavesPerBlock + wave;
  const uint64_t nwaves = (uint64_t)gridDim.x * kWavesPerBlock;
  const uint64_t n_steps = (n_blocks + kCountGroup - 1) / kCountGroup;
  const uint64_t n_vec = ((uintptr_t)sample % 16) == 0 ? n_blocks / kCountGroup : 0;
  uint32_t acc[NACC][P];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int j = 0; j < P; ++j) acc[a][j] = 0;
  for (uint64_t g = gwave; g < n_steps; g += nwaves) {
    uint32_t w[kCountWords];
    if (g < n_vec) {
      const uint4* q = reinterpret_cast<const uint4*>(sample) + g * (kCountGroup / 4) + lane;
#pragma unroll
      for (int j = 0; j < kCountWords / 4; ++j) {
        const uint4 v = q[j * kWave];
        w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
      }
    } else {
      const uint64_t base = g * kCountGroup + 4ull * lane;
#pragma unroll
      for (int j = 0; j < kCountWords / 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t k = base + 4ull * kWave * j + c;
          w[4 * j + c] = k < n_blocks ? sample[k] : 0u;
        }
    }
    if constexpr (NPOS == 32) {
      uint32_t s[6];
      sliced_count32(w, s);
      sliced_accumulate<P, 6>(acc[0], s);
    } else {
      uint32_t we[16], wo[16], se[5], so[5];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        we[2 * j] = w[4 * j];
        we[2 * j + 1] = w[4 * j + 2];
        wo[2 * j] = w[4 * j + 1];
        wo[2 * j + 1] = w[4 * j + 3];
      }
      sliced_count16(we, se);
      sliced_count16(wo, so);
      sliced_accumulate<P, 5>(acc[0], se);
      sliced_accumulate<P, 5>(acc[NACC - 1], so);
    }
  }
  // each lane's count is below 2^24 (at most kCountMaxSteps steps per wave),
  // so a wave's sum fits 32 bits
#pragma unroll
  for (int b = 0; b < NPOS; ++b) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) c += __builtin_amdgcn_ubfe(acc[b / 32][j], b % 32, 1) << j;
    const uint32_t t = wave_sum(c);
    if (lane == 0) part[wave][b] = t;
  }
  __syncthreads();
  if (threadIdx.x < NPOS) {
    unsigned long long t = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) t += part[w][threadIdx.x];
    partials[(uint64_t)threadIdx.x * gridDim.x + blockIdx.x] = t;
  }
}

// counts[b] = sum of column b of the transposed partials; one wave per
// position (launched as NPOS / 4 workgroups of 4 waves).
__global__ __launch_bounds__(kBlockThreads) void reduce_counts_kernel(
    const unsigned long long* __restrict__ partials, uint32_t n_parts,
    unsigned long long* __restrict__ counts) {
  const uint32_t lane = lane_id();
  const uint32_t b = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  const unsigned long long* col = partials + (uint64_t)b * n_parts;
  unsigned long long t0 = 0, t1 = 0, t2 = 0, t3 = 0;
  uint32_t i = lane;
  for (; i + 3 * kWave < n_parts; i += 4 * kWave) {
    t0 += col[i];
    t1 += col[i + kWave];
    t2 += col[i + 2 * kWave];
    t3 += col[i + 3 * kWave];
  }
  for (; i < n_parts; i += kWave) t0 += col[i];
  unsigned long long t = (t0 + t1) + (t2 + t3);
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) t += __shfl_xor(t, d, kWave);
  if (lane == 0) counts[b] = t;
}

// Flag bits of rows [base, base + k) (bit j of fl: row base + j is stored
// compressed), 1 <= k <= 64, written into their one or two flag words
// without assuming the words were cleared: the piece's bits are cleared with
// an atomic AND, then the set ones ORed in (one row alone: a single OR or
// AND).  No other piece touches these bits, so pieces that share a word
// commute.  The piece that ends the table also clears the bits of its word
// past the table (they must read 0).
__device__ __forceinline__ void put_flag_bits(unsigned long long* flags, uint64_t base,
                                              uint32_t k, unsigned long long fl,
                                              uint64_t n_rows) {
  const uint32_t sh = (uint32_t)(base & 63u);
  const uint32_t end = sh + k;  // one past the piece's last bit, counted from word 0
  const bool last = base + k == n_rows;
  unsigned long long* w0 = flags + (base >> 6);
  const unsigned long long tail = last && end < 64u ? ~0ull << end : 0ull;
  if (k == 1u) {  // rows compressed one per workgroup: one atomic per row
    if (fl & 1ull)
      atomicOr(w0, 1ull << sh);
    else
      atomicAnd(w0, ~(1ull << sh));
    if (tail) atomicAnd(w0, ~tail);
    return;
  }
  const unsigned long long span = k == 64u ? ~0ull : ((1ull << k) - 1ull);
  atomicAnd(w0, ~((span << sh) | tail));
  if (fl << sh) atomicOr(w0, fl << sh);
  if (end > 64u) {  // the piece continues in the next word (sh > 0 here)
    unsigned long long clear1 = span >> (64u - sh);
    if (last) clear1 |= ~0ull << (end - 64u);
    atomicAnd(w0 + 1, ~clear1);
    const unsigned long long set1 = fl >> (64u - sh);
    if (set1) atomicOr(w0 + 1, set1);
  }
}

// Flag bits of rows [base, base + k) written as whole bytes with plain
// stores, base a multiple of 8 and 1 <= k <= 64, by a whole wave (lane j
// writes byte j).  The caller owns every row of these bytes: k is a multiple
// of 8 or the piece ends the table, so no other piece shares a byte and no
// atomic is needed.  The piece that ends the table also zeroes the bytes of
// its word past the table (they must read 0).
__device__ __forceinline__ void put_flag_bytes(unsigned long long* flags, uint64_t base,
                                               uint32_t k, unsigned long long fl,
                                               uint64_t n_rows, uint32_t lane) {
  unsigned char* fb = reinterpret_cast<unsigned char*>(flags) + base / 8;
  const uint32_t nb = (k + 7u) / 8u;
  const uint32_t last =
      base + k == n_rows ? (uint32_t)((n_rows + 63u) / 64u * 8u - base / 8u) : nb;
  if (lane < last) fb[lane] = lane < nb ? (unsigned char)(fl >> (8u * lane)) : (unsigned char)0;
}

// [IBP] Compression, one workgroup per row.  The row's stream is assembled
// in LDS: header words from per-chunk ballots, a workgroup scan of the chunk
// match counts, then every lane ORs its payload (<= 2 words) into place with
// LDS atomics (OR commutes, so the bytes do not depend on timing), and the
// finished words are written out with coalesced stores.  A row whose stream
// would not be shorter than the raw row is copied raw.  In place (src ==
// slots) is safe: every read of a row happens before the barrier that
// precedes its first write.
template <int NR, uint32_t MAXW>
__global__ __launch_bounds__(kBlockThreads) void compress_kernel(
    Codec cd, uint64_t n_rows, const uint32_t* src, uint32_t* slots,
    unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits, int vec) {
  __shared__ uint32_t buf[MAXW + 4];
  __shared__ uint32_t chunk_pre[MAXW / kWave + 1];
  __shared__ uint32_t total_m;
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t n = cd.n;
  const uint32_t nchunks = (n + kWave - 1) / kWave;

  for (uint64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    const uint32_t* x_row = src + row * n;
    uint32_t* s_row = slots + row * n;

    for (uint32_t j = threadIdx.x; j < n + 4; j += kBlockThreads) buf[j] = 0;
    __syncthreads();

    // header bits and per-chunk match counts
    for (uint32_t c = wave; c < nchunks; c += kWavesPerBlock) {
      uint32_t k = c * kWave + lane;
      bool valid = k < n;
      uint32_t x = valid ? x_row[k] : 0u;
      bool match = valid && ((x & cd.mask) == cd.bitval);
      unsigned long long h = __ballot(match);
      if (lane == 0) {
        chunk_pre[c] = (uint32_t)__popcll(h);
        buf[2 * c] = (uint32_t)h;
        buf[2 * c + 1] = (uint32_t)(h >> 32);
      }
    }
    __syncthreads();

    // exclusive scan of the chunk counts
    if (wave == 0) {
      uint32_t carry = 0;
      for (uint32_t b0 = 0; b0 < nchunks; b0 += kWave) {
        uint32_t c = b0 + lane;
        uint32_t v = c < nchunks ? chunk_pre[c] : 0u;
        uint32_t inc = wave_inclusive_scan(v, lane);
        if (c < nchunks) chunk_pre[c] = carry + inc - v;
        carry += __shfl(inc, kWave - 1, kWave);
      }
      if (lane == 0) total_m = carry;
    }
    __syncthreads();

    const uint32_t m = total_m;
    const uint32_t c_bits = n + 32u * n - cd.p * m;
    const bool flag = c_bits < 32u * n;

    if (!flag) {
      if (vec) {
        const uint4* a = reinterpret_cast<const uint4*>(x_row);
        uint4* o = reinterpret_cast<uint4*>(s_row);
        for (uint32_t j = threadIdx.x; j < n / 4; j += kBlockThreads) o[j] = a[j];
      } else {
        for (uint32_t j = threadIdx.x; j < n; j += kBlockThreads) s_row[j] = x_row[j];
      }
    } else {
      for (uint32_t c = wave; c < nchunks; c += kWavesPerBlock) {
        uint32_t k = c * kWave + lane;
        bool valid = k < n;
        uint32_t x = valid ? x_row[k] : 0u;
        bool match = valid && ((x & cd.mask) == cd.bitval);
        unsigned long long h = __ballot(match);
        uint32_t pre = chunk_pre[c] + bits_below_lane((uint32_t)h, (uint32_t)(h >> 32));
        if (valid) {
          uint32_t off = n + 32u * k - cd.p * pre;
          uint32_t len = match ? 32u - cd.p : 32u;
          uint32_t pay = match ? extract_kept<NR>(x, cd.runs) : x;
          if (len) {
            uint32_t sh = off & 31u, wi = off >> 5;
            atomicOr(&buf[wi], pay << sh);
            if (sh + len > 32u) atomicOr(&buf[wi + 1], pay >> (32u - sh));
          }
        }
      }
      __syncthreads();
      const uint32_t nw = (c_bits + 31u) >> 5;
      for (uint32_t j = threadIdx.x; j < nw; j += kBlockThreads) __builtin_nontemporal_store(buf[j], &s_row[j]);
    }
    if (threadIdx.x == 0) {
      put_flag_bits(flags, row, 1u, flag ? 1ull : 0ull, n_rows);
      if (row_bits) row_bits[row] = c_bits;
    }
    // the LDS stream is reused only by a next row; after the last one the
    // workgroup ends without waiting for its stores (a barrier would)
    if (row + gridDim.x < n_rows) __syncthreads();
  }
}

// One tensor of a batched compression launch (compress_wg_kernel).
constexpr uint32_t kCompressBatchMax = 16;
struct CompressTensor {
  const uint32_t* src;
  uint32_t* slots;
  unsigned long long* flags;
  uint32_t* row_bits;
  uint64_t n_rows;
  uint32_t pad;  // stored rows padded to 64-byte units (device slots)
  uint32_t unused;
};
struct CompressBatch {
  uint32_t count;
  uint32_t unused;
  uint32_t wg_end[kCompressBatchMax];  // workgroups of tensors [0, t]
  CompressTensor t[kCompressBatchMax];
};

// [IBP] Compression of rows of exactly WPB * 64 * CPW blocks (the long rows
// of LLM weight matrices), a workgroup of WPB waves per row: each wave holds
// its share of the row in registers (chunks wave * CPW ... + CPW - 1, one
// block per lane each), so the row is read once.  A workgroup takes a
// contiguous range of `per_wg` rows (at most 64) and loads its next row while
// it encodes one.  The chunk ballots are the header words (each placed
// in its lane with a lane write); the waves' match totals, exchanged through
// LDS, give each wave its carry; payloads are ORed into the workgroup's LDS
// stream, which is then written with coalesced stores (a raw row straight
// from the registers).  Three barriers per row.  The range's flag bits are
// written once at its end: as whole bytes with plain stores when per_wg is a
// multiple of 8 (the workgroup owns those bytes), else with an atomic AND and
// OR; per-row atomics on the few flag words of a matrix serialize (one per
// row cost a third of the time of a 4096 x 8 KiB matrix).  In place
// (src == slots) is safe: every wave has read its part of the row before the
// first barrier and nothing is written before it, and the rows loaded ahead
// are other rows, whose slots no store of this one touches.  One launch
// takes up to kCompressBatchMax tensors of the same row length (the matrices
// of a layer): each workgroup finds its tensor from the running workgroup
// counts, and no range spans two tensors.
template <int NR, int CPW, int WPB>
__global__ __launch_bounds__(WPB * kWave) void compress_wg_kernel(Codec cd, CompressBatch batch,
                                                                  uint32_t per_wg) {
  constexpr uint32_t n = (uint32_t)CPW * kWave * WPB;
  uint32_t t = 0;
  while (blockIdx.x >= batch.wg_end[t]) ++t;
  const CompressTensor& ct = batch.t[t];
  const uint64_t n_rows = ct.n_rows;
  const uint32_t* src = ct.src;
  uint32_t* slots = ct.slots;
  unsigned long long* flags = ct.flags;
  uint32_t* row_bits = ct.row_bits;
  const uint32_t wg = blockIdx.x - (t ? batch.wg_end[t - 1] : 0u);  // within the tensor
  // the row's stream and the waves' match totals; with two of each (rows of
  // 8 KiB, whose two streams fit beside the other resident workgroups'),
  // consecutive rows alternate between them and a row needs no barrier
  // after its stores: the next use of a buffer is two rows on, past both
  // barriers of the row between
  constexpr int NB = CPW == 8 ? 2 : 1;
  __shared__ uint32_t buf_all[NB][n + 4];
  __shared__ uint32_t wtot_all[NB][WPB];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t c0 = wave * CPW;  // the wave's first chunk
  const uint32_t lane_byte = (c0 * kWave + lane) * 4u;
  // a run's kept bits at their payload position: extract = OR of
  // (x >> shift) & kept, a shift and an and-or per run
  constexpr int NK = NR > 0 ? NR : 1;
  uint32_t kept[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) kept[j] = NR > 0 ? cd.runs.place[j] >> cd.runs.shift[j] : 0u;
  // this lane's first payload offset in bits, less the carry: the stream's
  // n header bits, then 32 bits per block before it
  const uint32_t off0 = n + 8u * lane_byte;
  const int negp = -(int)cd.p;
  const uint64_t r0 = (uint64_t)wg * per_wg;
  const uint64_t r1 = min(n_rows, r0 + per_wg);
  // a row past the range loads as zeros (empty range), never out of bounds
  auto load = [&](uint32_t (&v)[CPW], uint64_t r) {
    const __amdgpu_buffer_rsrc_t in =
        row_rsrc(src + (r < r1 ? r : r0) * n, r < r1 ? n * 4u : 0u);
    // the lane's offset as an opaque value: the chunks' offsets are then
    // immediates on it, not CPW precomputed registers
    uint32_t lb = lane_byte;
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      v[c] = __builtin_amdgcn_raw_buffer_load_b32(in, lb + c * kWave * 4u, 0, kRowLoad);
  };
  uint32_t x[CPW];
  load(x, r0);
  unsigned long long fl = 0;  // bit j: row r0 + j is stored compressed
  for (uint64_t row = r0; row < r1; ++row) {
    uint32_t* s_row = slots + row * n;
    uint32_t* buf = buf_all[NB == 2 ? (uint32_t)(row - r0) & 1u : 0u];
    uint32_t* wtot = wtot_all[NB == 2 ? (uint32_t)(row - r0) & 1u : 0u];
    uint32_t y[CPW];  // the next row, in flight
    load(y, row + 1);
    uint32_t mw = 0;
    uint32_t hword = 0;  // lane 2c / 2c + 1: low / high half of chunk c's ballot
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const unsigned long long h = __ballot((x[c] & cd.mask) == cd.bitval);
      mw += (uint32_t)__popcll(h);
      hword = (uint32_t)lane_write((int)(uint32_t)h, 2 * c, (int)hword);
      hword = (uint32_t)lane_write((int)(uint32_t)(h >> 32), 2 * c + 1, (int)hword);
    }
    // the payload part of the stream starts zeroed (16-byte LDS stores: n/32
    // and n + 4 are multiples of 4); header words are whole
    {
      u32x4* b4 = reinterpret_cast<u32x4*>(buf);
      for (uint32_t j = n / 128 + threadIdx.x; j < (n + 4) / 4; j += WPB * kWave)
        b4[j] = u32x4{0u, 0u, 0u, 0u};
    }
    if (lane < 2u * CPW) buf[2u * c0 + lane] = hword;
    if (lane == 0) wtot[wave] = mw;
    __syncthreads();
    uint32_t carry = 0, m = 0;
#pragma unroll
    for (int w = 0; w < WPB; ++w) {
      const uint32_t t = wtot[w];
      carry += (uint32_t)w < wave ? t : 0u;
      m += t;
    }
    const uint32_t c_bits = n + 32u * n - cd.p * m;
    const bool flag = c_bits < 32u * n;
    fl |= (unsigned long long)flag << (row - r0);
    if (flag) {
      // off0 as an opaque value of this row: folded into CPW loop-invariant
      // chunk bases it would hold as many registers
      uint32_t ob = off0;
      asm volatile("" : "+v"(ob));
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        // the match test again: two instructions, where reusing the first
        // pass's masks keeps CPW of them in scalar registers and costs as
        // many to turn back into lane masks
        asm volatile("" : "+v"(x[c]));
        const bool match = (x[c] & cd.mask) == cd.bitval;
        const unsigned long long h = __ballot(match);
        // offset = this lane's 32-bit slots before it less p per stripped
        // block before it: one multiply-add on the lane's count and a scalar
        // for the chunk (kept opaque so that it is not split into per-chunk
        // vector constants)
        const uint32_t below = bits_below_lane((uint32_t)h, (uint32_t)(h >> 32));
        uint32_t t = (uint32_t)(c * kWave * 32) - cd.p * carry;
        asm volatile("" : "+s"(t));
        const uint32_t off = (uint32_t)mul_i24((int)below, negp) + ob + t;
        if constexpr (NR != 0) {
          // p < 32: every block has a payload of 32 - p or 32 bits; its two
          // stream words get their bits with no branch (the second OR is of
          // zero when the payload ends in the first word)
          uint32_t e;
          if constexpr (NR > 0) {
            e = (x[c] >> cd.runs.shift[0]) & kept[0];
#pragma unroll
            for (int j = 1; j < NR; ++j) e |= (x[c] >> cd.runs.shift[j]) & kept[j];
          } else {
            e = extract_kept<NR>(x[c], cd.runs);
          }
          const uint32_t pay = match ? e : x[c];
          const unsigned long long w2 = (unsigned long long)pay << (off & 31u);
          atomicOr(&buf[off >> 5], (uint32_t)w2);
          atomicOr(&buf[(off >> 5) + 1u], (uint32_t)(w2 >> 32));
        } else {
          // p = 32: a stripped block has no payload
          if (!match) {
            const uint32_t sh = off & 31u, wi = off >> 5;
            atomicOr(&buf[wi], x[c] << sh);
            if (sh) atomicOr(&buf[wi + 1], x[c] >> (32u - sh));
          }
        }
        carry += (uint32_t)__popcll(h);
      }
    }
    __syncthreads();
    if (!flag) {
      const __amdgpu_buffer_rsrc_t out = row_rsrc(s_row, n * 4u);
      uint32_t lb = lane_byte;
      asm volatile("" : "+v"(lb));
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        __builtin_amdgcn_raw_buffer_store_b32(x[c], out, lb + c * kWave * 4u, 0, kRowStore);
    } else {
      const uint32_t nw = store_words(s_row, (c_bits + 31u) >> 5, n, ct.pad);
      uint32_t j0 = 0;
      if ((reinterpret_cast<uintptr_t>(s_row) & 15u) == 0) {  // whole 16-byte units
        const u32x4* b4 = reinterpret_cast<const u32x4*>(buf);
        u32x4* o4 = reinterpret_cast<u32x4*>(s_row);
        for (uint32_t j = threadIdx.x; j < nw / 4; j += WPB * kWave) __builtin_nontemporal_store(b4[j], &o4[j]);
        j0 = nw & ~3u;
      }
      for (uint32_t j = j0 + threadIdx.x; j < nw; j += WPB * kWave) __builtin_nontemporal_store(buf[j], &s_row[j]);
    }
    if (threadIdx.x == 0 && row_bits) row_bits[row] = c_bits;
#pragma unroll
    for (int c = 0; c < CPW; ++c) x[c] = y[c];
    // the LDS stream is reused only by a next row; after the last one the
    // workgroup ends without waiting for its stores (a barrier would)
    if (NB == 1 && row + 1 < r1) __syncthreads();
  }
  if (wave == 0 && r0 < r1) {
    const uint32_t k = (uint32_t)(r1 - r0);
    if (per_wg % 8u == 0)
      put_flag_bytes(flags, r0, k, fl, n_rows, lane);
    else if (lane == 0)
      put_flag_bits(flags, r0, k, fl, n_rows);
  }
}

// Rows of one compressing wave: a contiguous range, as long for every wave
// of the launch (wpb waves per workgroup), taken in pieces of up to 64 rows.
// encode(row) compresses a row and returns its C; a row is stored compressed
// when C < raw_bits.  A piece's flag bits are ORed into their one or two flag
// words at once, and its C values stored with one instruction.
template <typename Encode>
__device__ __forceinline__ void compress_row_range(uint64_t n_rows, uint32_t wave, uint32_t wpb,
                                                   uint32_t raw_bits,
                                                   unsigned long long* __restrict__ flags,
                                                   uint32_t* __restrict__ row_bits,
                                                   Encode encode) {
  const uint32_t lane = lane_id();
  const uint64_t waves = (uint64_t)gridDim.x * wpb;
  const uint64_t per = (n_rows + waves - 1) / waves;
  const uint64_t r0 = min(n_rows, ((uint64_t)blockIdx.x * wpb + wave) * per);
  const uint64_t r1 = min(n_rows, r0 + per);
  for (uint64_t base = r0; base < r1; base += 64) {
    const uint32_t K = (uint32_t)min<uint64_t>(64, r1 - base);
    uint32_t cb = 0u;              // lane k: C of row k of the piece
    unsigned long long fl = 0ull;  // bit k: row k stored compressed
    for (uint32_t k = 0; k < K; ++k) {
      const uint32_t c_bits = encode(base + k);
      cb = lane == k ? c_bits : cb;
      fl |= (unsigned long long)(c_bits < raw_bits) << k;
    }
    if (row_bits && lane < K) row_bits[base + lane] = cb;
    if (lane == 0) put_flag_bits(flags, base, K, fl, n_rows);
  }
}

// [IBP] Compression of rows of exactly 64*NCH blocks, one wave per row.  A
// wave takes a contiguous range of rows (the launch gives every wave the
// same number), in pieces of up to 64 rows whose flag bits it ORs into their
// flag words at once and whose C values it stores with one instruction.  A
// row is read into registers (NCH blocks per lane); each chunk's match
// ballot is its 64-bit header word (placed in its lane with a lane write),
// the chunk prefixes are a scalar running sum, and the payloads are ORed into
// a wave-private LDS stream buffer, written out with NCH buffer stores whose
// range is the row's stored words (the same instructions for a raw row).  No
// workgroup barriers.  In place (src == slots) is safe: a row's stores depend
// on all of its loads, and no other row's stores touch it.
template <int NR, int NCH>
__global__ __launch_bounds__(kBlockThreads) void compress_rows_kernel(
    Codec cd, uint64_t n_rows, const uint32_t* src, uint32_t* slots,
    unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits) {
  __shared__ uint32_t lds_all[kWavesPerBlock][NCH * kWave + 4];
  constexpr uint32_t n = (uint32_t)NCH * kWave;
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds_all[wave];
  constexpr int NK = NR > 0 ? NR : 1;
  uint32_t kept[NK];  // a run's kept bits at their payload position
#pragma unroll
  for (int j = 0; j < NK; ++j) kept[j] = NR > 0 ? cd.runs.place[j] >> cd.runs.shift[j] : 0u;
  const int negp = -(int)cd.p;
  compress_row_range(n_rows, wave, kWavesPerBlock, 32u * n, flags, row_bits, [&](uint64_t row) {
    uint32_t x[NCH];
    {
      const __amdgpu_buffer_rsrc_t in = row_rsrc(src + row * n, n * 4u);
      uint32_t lb = lane * 4u;  // opaque: the chunks' offsets are immediates on it
      asm volatile("" : "+v"(lb));
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        x[c] = __builtin_amdgcn_raw_buffer_load_b32(in, lb + c * kWave * 4u, 0, kRowLoad);
    }
    uint32_t m = 0;
    uint32_t hword = 0;  // lane 2c / 2c + 1: low / high half of chunk c's ballot
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const unsigned long long h = __ballot((x[c] & cd.mask) == cd.bitval);
      m += (uint32_t)__popcll(h);
      hword = (uint32_t)lane_write((int)(uint32_t)h, 2 * c, (int)hword);
      hword = (uint32_t)lane_write((int)(uint32_t)(h >> 32), 2 * c + 1, (int)hword);
    }
    const uint32_t c_bits = n + 32u * n - cd.p * m;
    const bool flag = c_bits < 32u * n;
    uint32_t words = n;
    if (flag) {
      words = store_words(slots + row * n, (c_bits + 31u) >> 5, n, cd.pad);
      for (uint32_t j = n / 32 + lane; j < words + 1; j += kWave) buf[j] = 0u;
      if (lane < 2 * NCH) buf[lane] = hword;
      wave_lds_sync();
      uint32_t ob = n + 32u * lane;  // opaque, as the load offsets
      asm volatile("" : "+v"(ob));
      uint32_t carry = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        // the match test again (two instructions, where keeping NCH ballots
        // in scalar registers costs as many to turn back into lane masks)
        asm volatile("" : "+v"(x[c]));
        const bool match = (x[c] & cd.mask) == cd.bitval;
        const unsigned long long h = __ballot(match);
        const uint32_t below = bits_below_lane((uint32_t)h, (uint32_t)(h >> 32));
        uint32_t t = (uint32_t)(c * kWave * 32) - cd.p * carry;
        asm volatile("" : "+s"(t));
        const uint32_t off = (uint32_t)mul_i24((int)below, negp) + ob + t;
        uint32_t e;
        if constexpr (NR > 0) {
          e = (x[c] >> cd.runs.shift[0]) & kept[0];
#pragma unroll
          for (int j = 1; j < NR; ++j) e |= (x[c] >> cd.runs.shift[j]) & kept[j];
        } else {
          e = extract_kept<NR>(x[c], cd.runs);
        }
        const uint32_t pay = match ? e : x[c];
        // the payload's bits in its first word and the next (zero when it
        // ends in the first).  With p = 32 a matched block has no payload,
        // and only the other lanes take part (many empty payloads at one
        // offset would all hit one LDS word); otherwise no branch.
        const unsigned long long w2 = (unsigned long long)pay << (off & 31u);
        if (NR != 0 || !match) {
          atomicOr(&buf[off >> 5], (uint32_t)w2);
          atomicOr(&buf[(off >> 5) + 1u], (uint32_t)(w2 >> 32));
        }
        carry += (uint32_t)__popcll(h);
      }
      wave_lds_sync();
#pragma unroll
      for (int c = 0; c < NCH; ++c) x[c] = c * kWave < words ? buf[c * kWave + lane] : 0u;
    }
    const __amdgpu_buffer_rsrc_t out = row_rsrc(slots + row * n, words * 4u);
    uint32_t lb = lane * 4u;
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      __builtin_amdgcn_raw_buffer_store_b32(x[c], out, lb + c * kWave * 4u, 0, kRowStore);
    wave_lds_sync();
    return c_bits;
  });
}

// [IBP] Decompression.  One wave per task = (output row, segment of `seg`
// blocks, seg a multiple of 64 and at most kSegBlocks).  For a compressed row
// the wave
//   1. counts the stripped blocks before its segment (popcount of header
//      words) and inside it,
//   2. fetches the segment's stream words [a/32, ceil(b/32)) into its LDS
//      window with coalesced 16-byte loads,
//   3. per 64-block chunk: header word -> per-lane bit offset (mbcnt + carry)
//      -> two LDS words -> funnel shift -> deposit + Bitval -> store.
// A raw row is a straight copy.
// One decode task: segment s (blocks [s*seg, min(n, s*seg + seg))) of output
// row i, whose source is row ids[i] of the image (row i for a full
// decompress).  Rows of n blocks; `lds` is the wave's window.
template <int MODE, int NR>
__device__ __forceinline__ void decode_segment_task(
    const Codec& cd, uint32_t n, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    const uint32_t* __restrict__ arena, const unsigned long long* __restrict__ cache_loc,
    uint64_t n_rows, uint64_t i, uint32_t s, uint32_t seg, uint32_t* __restrict__ dst, int vec,
    uint32_t* lds, uint32_t lane) {
  const uint64_t id = MODE != kModeTable ? (uint64_t)ids[i] : i;
  uint32_t* out = dst + i * n;
  const uint32_t lo = s * seg;
  const uint32_t hi = min(n, lo + seg);
  if (MODE != kModeTable && id >= n_rows) {  // an id outside the table gives a zero row
    for (uint32_t j = lo + lane; j < hi; j += kWave) out[j] = 0u;
    return;
  }
  const unsigned long long loc = MODE == kModeCached ? cache_loc[id] : 0ull;
  const unsigned long long fw = (loc & IBP_LOC_RESIDENT) ? 0ull : flags[id >> 6];
  const uint32_t* src = row_source<MODE>(slots, arena, id, n, loc);
  const uint32_t lim = row_words<MODE>(n, loc);
  const bool flag = row_flag<MODE>(fw, id, loc);

  // The header words are requested together with the flag word (for a raw
  // row they are row data inside the slot, read and then ignored): the
  // segment's words one per lane, and the words before it, whose stripped
  // count is the segment's carry, in batches of four per lane.
  const uint32_t hw_n = (hi - lo + 31) / 32;
  uint32_t hw = 0;
  if (lane < hw_n) hw = src[lo / 32 + lane];
  uint32_t acc = 0;
  for (uint32_t t0 = 0; t0 < lo / 32; t0 += 4 * kWave) {
    uint32_t w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = src[min(t0 + c * kWave + lane, lo / 32 - 1)];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc += t0 + c * kWave + lane < lo / 32 ? __popc(w[c]) : 0u;
  }

  if (!flag) {
    if (vec) {
      const uint4* a = reinterpret_cast<const uint4*>(src);
      uint4* o = reinterpret_cast<uint4*>(out);
      for (uint32_t j = lo / 4 + lane; j < hi / 4; j += kWave) o[j] = a[j];
    } else {
      for (uint32_t j = lo + lane; j < hi; j += kWave) out[j] = src[j];
    }
    return;
  }

  // stripped blocks before the segment: header words [0, lo/32) (all header)
  const uint32_t carry = lo ? wave_sum(acc) : 0u;
  // the segment's header words, one per lane; bits at or past n belong to
  // the payloads and are cleared
  if (lane < hw_n) {
    const uint32_t valid_bits = min(32u, hi - 32u * (lo / 32 + lane));
    if (valid_bits < 32u) hw &= (1u << valid_bits) - 1u;
  }
  const uint32_t m_seg = wave_sum(__popc(hw));

  // stream bit range of the segment's payloads, and its LDS window
  // (for an image that ibp_compress wrote, wb <= ceil(C/32) <= n; the
  // clamps only keep a corrupt header from reading past the slot or entry)
  const uint32_t a = n + 32u * lo - cd.p * carry;
  const uint32_t b = n + 32u * hi - cd.p * (carry + m_seg);
  const uint32_t wb = min((b + 31u) >> 5, lim);
  const uint32_t wa = min(a >> 5, wb);
  uint32_t base;
  if (vec) {
    base = wa & ~3u;
    stage_window<5, MODE != kModeCached>(reinterpret_cast<const u32x4*>(src + base),
                                         reinterpret_cast<u32x4*>(lds), (wb - base + 3u) / 4u,
                                         lane);
  } else {
    base = wa;
    stage_window<4, MODE != kModeCached>(src + wa, lds, wb - wa, lane);
  }
  wave_lds_sync();

  // u = bit offset, relative to the LDS window, of the payload of the
  // chunk's first block; lane l's payload starts 32*l - p*(stripped blocks
  // of the chunk below l) further on.
  uint32_t u = n + 32u * lo - cd.p * carry - 32u * base;
  const uint32_t l32 = lane * 32u;
  const int negp = -(int)cd.p;
  // the lane's bit cursor (u plus 32 bits per lane below it) in a vector
  // register, advanced by one add per chunk
  uint32_t ul = u + l32;
  auto chunk = [&](uint32_t k0) {  // a whole 64-block chunk
    const uint32_t q = (k0 - lo) / 32;
    const uint32_t h_lo = __builtin_amdgcn_readlane(hw, q);
    const uint32_t h_hi = __builtin_amdgcn_readlane(hw, q + 1);
    const uint32_t rel = (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + ul;
    // the window word index as an opaque value: its LDS address is one
    // shift-add on it, not a shift, an and and an add on rel
    uint32_t wi = __builtin_amdgcn_ubfe(rel, 5, 27);
    asm volatile("" : "+v"(wi));
    const uint32_t v = __builtin_amdgcn_alignbit(lds[wi + 1], lds[wi], rel & 31u);
    const bool stripped =
        __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
    const uint32_t x = stripped ? deposit_kept<NR>(v, cd.runs, cd.bitval) : v;
    __builtin_nontemporal_store(x, out + k0 + lane);
    uint32_t adv =
        32u * kWave - cd.p * (uint32_t)__popcll(((unsigned long long)h_hi << 32) | h_lo);
    asm volatile("" : "+s"(adv));
    ul += adv;
    u += adv;
  };
  const uint32_t full_hi = lo + ((hi - lo) & ~(uint32_t)(kWave - 1));
  uint32_t k0 = lo;
  if (hi - lo == kSegBlocks) {  // a whole segment: unrolled
#pragma unroll
    for (uint32_t c = 0; c < kSegBlocks / kWave; ++c) chunk(lo + c * kWave);
    k0 = hi;
  } else {
    for (; k0 < full_hi; k0 += kWave) chunk(k0);
  }
  if (k0 < hi) {  // ragged end of the row (n not a multiple of 64)
    const uint32_t q = (k0 - lo) / 32;
    const uint32_t h_lo = __builtin_amdgcn_readlane(hw, q);
    const uint32_t h_hi = __builtin_amdgcn_readlane(hw, q + 1);
    const bool valid = k0 + lane < hi;
    const uint32_t rel = valid ? u + l32 - __umul24(cd.p, bits_below_lane(h_lo, h_hi)) : 0u;
    const uint32_t x = decode_block<NR>(lds, rel, h_lo, h_hi, cd);
    if (valid) out[k0 + lane] = x;
  }
  wave_lds_sync();
}

template <int MODE, int NR>
__global__ __launch_bounds__(kBlockThreads) void decode_segments_kernel(
    Codec cd, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    const uint32_t* __restrict__ arena, const unsigned long long* __restrict__ cache_loc,
    uint64_t n_rows, uint64_t n_tasks, uint32_t nseg, uint32_t seg, uint32_t* __restrict__ dst,
    int vec, int remap) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerBlock][kSegLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint32_t g = gridDim.x;
  for (uint64_t wg = remap ? xcd_remap(blockIdx.x, g) : blockIdx.x; ; wg += g) {
    const uint64_t task = wg * kWavesPerBlock + wave;
    if (task >= n_tasks) break;
    const uint64_t i = task / nseg;
    const uint32_t s = (uint32_t)(task - i * nseg);
    decode_segment_task<MODE, NR>(cd, cd.n, slots, flags, ids, arena, cache_loc, n_rows, i, s,
                                  seg, dst, vec, lds, lane);
  }
}

// [IBP] Decompression of several tensors that share one Mask/Bitval (the
// layers of a model are decompressed tensor group by tensor group) in one
// launch: the segment tasks of every tensor, one after the other, each
// mapped to its tensor by the running task counts.  One launch instead of
// one per tensor keeps the GPU full across tensor boundaries.
constexpr uint32_t kBatchMax = 16;
struct BatchTensor {
  const uint32_t* slots;
  const unsigned long long* flags;
  uint32_t* dst;
  uint32_t n;     // blocks per row
  uint32_t nseg;  // segments per row
  uint32_t vec;   // 16-byte aligned rows and buffers
  uint32_t nw;    // 32-bit words per row
};
struct Batch {
  uint32_t count;
  uint32_t pad;
  uint64_t end[kBatchMax];  // tasks of tensors [0, t]
  BatchTensor t[kBatchMax];
};

template <int NR>
__global__ __launch_bounds__(kBlockThreads) void decode_batch_kernel(Codec cd, Batch batch) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerBlock][kSegLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint64_t n_tasks = batch.end[batch.count - 1];
  const uint32_t g = gridDim.x;
  for (uint64_t wg = blockIdx.x; ; wg += g) {
    const uint64_t task = wg * kWavesPerBlock + wave;
    if (task >= n_tasks) break;
    uint32_t t = 0;
    while (task >= batch.end[t]) ++t;
    const BatchTensor& bt = batch.t[t];
    const uint64_t local = task - (t ? batch.end[t - 1] : 0ull);
    const uint64_t i = local / bt.nseg;
    const uint32_t s = (uint32_t)(local - i * bt.nseg);
    decode_segment_task<kModeTable, NR>(cd, bt.n, bt.slots, bt.flags, nullptr, nullptr, nullptr,
                                        0, i, s, kSegBlocks, bt.dst, (int)bt.vec, lds, lane);
  }
}

// [IBP] Decompression of short rows (n <= kSegBlocks blocks: one task per
// row), software pipelined across the rows a wave handles.  The first
// kSpecWords words of a slot hold the whole participation header (n/32 <= 32
// words) and, for well compressed rows, often the whole stream; so while the
// wave decodes row j it already has in flight the id of row j+2 and the flag
// word and first slot words of row j+1 (kept in one VGPR).
//
// One hardware counter tracks a wave's loads and stores together, so a wait
// for the prefetched window can only spare the stores issued after it if
// their number is known when the kernel is compiled.  With NCH > 0 (rows of
// exactly 64*NCH blocks) every row path issues exactly NCH stores after the
// prefetch, the decode is fully unrolled, and the first window is waited for
// before the loop: the wait at the top of the loop then leaves the previous
// row's stores in flight.  NCH == 0 handles any n.  n_out < 2^31 (the host
// splits larger gathers).
template <int MODE, int NR, int NCH>
__global__ __launch_bounds__(kBlockThreads) void decode_rows_kernel(
    Codec cd, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    const uint32_t* __restrict__ arena, const unsigned long long* __restrict__ cache_loc,
    uint64_t n_rows, uint32_t n_out, uint32_t* __restrict__ dst, int vec) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerBlock][kSegLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint32_t n = NCH > 0 ? (uint32_t)NCH * kWave : cd.n;
  const uint32_t spec = min(n, kSpecWords);
  const uint32_t hw_n = (n + 31) / 32;
  const uint32_t stride = gridDim.x * kWavesPerBlock;
  const uint32_t keep_bits = 32u - cd.p;
  const uint32_t lane_keep = lane * keep_bits;
  const int negp = -(int)cd.p;
  const uint32_t l32 = 32u * lane;
  const uint32_t full = n & ~(uint32_t)(kWave - 1);

  uint32_t i = blockIdx.x * kWavesPerBlock + wave;
  if (i >= n_out) return;

  auto row_id = [&](uint32_t r) -> uint64_t { return MODE != kModeTable ? (uint64_t)ids[r] : r; };
  auto in_table = [&](uint64_t id) -> bool { return MODE == kModeTable || id < n_rows; };

  // With the cache a row's window depends on its locator, one load further
  // down the chain: the locator of row j+1 is requested at the top of the
  // iteration for row j, before this row's stream is staged.
  uint64_t id = row_id(i);
  unsigned long long loc = (MODE == kModeCached && in_table(id)) ? cache_loc[id] : 0ull;
  unsigned long long fw = in_table(id) ? flags[id >> 6] : 0ull;
  uint32_t win = (in_table(id) && lane < min(spec, row_words<MODE>(n, loc)))
                     ? row_source<MODE>(slots, arena, id, n, loc)[lane] : 0u;
  uint64_t id_next = (i + stride < n_out) ? row_id(i + stride) : 0;
  asm volatile("" ::"v"(win));  // the first window is waited for here, not in the loop

  while (true) {
    const uint32_t i_next = i + stride;
    const bool have_next = i_next < n_out;
    const uint64_t id_after = (have_next && i_next + stride < n_out) ? row_id(i_next + stride) : 0;
    unsigned long long loc_next = 0;
    if constexpr (MODE == kModeCached)
      if (have_next && in_table(id_next)) loc_next = cache_loc[id_next];
    uint32_t* out = dst + (uint64_t)i * n;
    const uint32_t* src = row_source<MODE>(slots, arena, id, n, loc);
    const uint32_t lim = row_words<MODE>(n, loc);
    const bool valid_id = in_table(id);
    const bool flag = valid_id && row_flag<MODE>(fw, id, loc);

    // with NCH > 0 a raw row is staged in LDS like a stream, so that its
    // copy out issues no loads after the prefetch below
    if (flag || (NCH > 0 && valid_id)) {
      uint32_t wb = lim;
      if (flag) {
        // header words are lanes [0, hw_n) of the window; bits at or past n
        // belong to the payloads
        uint32_t hw = lane < hw_n ? win : 0u;
        if (lane == hw_n - 1 && (n & 31u)) hw &= (1u << (n & 31u)) - 1u;
        const uint32_t m = wave_sum(__popc(hw));
        wb = min((n + 32u * n - cd.p * m + 31u) >> 5, lim);
      }
      if (lane < spec) lds[lane] = win;
      if (wb > spec) {  // the rest of the stream
        // one batch: n <= 64 * NCH words (<= 1024 for NCH == 0) past the window
        constexpr int kV = NCH >= 8 ? NCH / 4 : (NCH > 0 ? 1 : 4);
        if (vec)
          stage_window<kV, MODE != kModeCached>(
              reinterpret_cast<const u32x4*>(src) + spec / 4,
              reinterpret_cast<u32x4*>(lds) + spec / 4, (wb + 3u) / 4u - spec / 4, lane);
        else
          stage_window<4, MODE != kModeCached>(src + spec, lds + spec, wb - spec, lane);
      }
      wave_lds_sync();
    }

    // next row's flag word and window: in flight while this row is decoded
    unsigned long long fw_next = 0;
    uint32_t win_next = 0;
    if (have_next && in_table(id_next)) {
      fw_next = flags[id_next >> 6];
      win_next = lane < min(spec, row_words<MODE>(n, loc_next))
                     ? row_source<MODE>(slots, arena, id_next, n, loc_next)[lane] : 0u;
    }

    if constexpr (NCH > 0) {
      // exactly NCH stores on every path
      uint32_t x[NCH];
      if (!flag) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) x[c] = valid_id ? lds[c * kWave + lane] : 0u;
      } else if constexpr (NR == 0) {
        // p = 32: a stripped block is Bitval and every other payload is one
        // whole stream word (n is a multiple of 64, so payloads stay word
        // aligned): word index = header words + unstripped blocks before it
        uint32_t uw = n / 32;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
          const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
          // 64-bit scalar ops on the header word (one s_not_b64, one s_bcnt1_b64)
          const unsigned long long h = ((unsigned long long)h_hi << 32) | h_lo;
          const unsigned long long kept = ~h;
          const uint32_t v = lds[bits_below_lane_acc((uint32_t)kept, (uint32_t)(kept >> 32), uw)];
          x[c] = __builtin_amdgcn_inverse_ballot_w64(h) ? cd.bitval : v;
          uw += (uint32_t)__popcll(kept);
        }
      } else {
        uint32_t u = n;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
          const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
          const uint32_t rel = (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + (u + l32);
          x[c] = decode_block<NR>(lds, rel, h_lo, h_hi, cd);
          u += 32u * kWave - cd.p * (uint32_t)__popcll(((unsigned long long)h_hi << 32) | h_lo);
        }
      }
      // the restored rows are streamed out: non-temporal stores
#pragma unroll
      for (int c = 0; c < NCH; ++c) __builtin_nontemporal_store(x[c], out + c * kWave + lane);
      // keep the stores ahead of the hand-over of the next window, so that
      // waiting for it can leave them in flight
      __builtin_amdgcn_sched_barrier(0);
      wave_lds_sync();
    } else if (!valid_id) {
      for (uint32_t j = lane; j < n; j += kWave) out[j] = 0u;
    } else if (!flag) {
      if (vec) {
        const uint4* a = reinterpret_cast<const uint4*>(src);
        uint4* o = reinterpret_cast<uint4*>(out);
        for (uint32_t j = lane; j < n / 4; j += kWave) o[j] = a[j];
      } else {
        for (uint32_t j = lane; j < n; j += kWave) out[j] = src[j];
      }
    } else {
      // u: stream bit offset of the payload of the current chunk's first
      // block.  Lane l's payload starts l*(32-p) + p*(unstripped blocks of the
      // chunk below l) further on.
      uint32_t u = n;
      uint32_t k0 = 0;
      for (; k0 < full; k0 += kWave) {
        const uint32_t q = k0 / 32;
        const uint32_t h_lo = __builtin_amdgcn_readlane(win, q);
        const uint32_t h_hi = __builtin_amdgcn_readlane(win, q + 1);
        const uint32_t rel = u + lane_keep + __umul24(cd.p, bits_below_lane(~h_lo, ~h_hi));
        uint32_t* o = out + k0;
        o[lane] = decode_block<NR>(lds, rel, h_lo, h_hi, cd);
        u += 32u * kWave - cd.p * (__popc(h_lo) + __popc(h_hi));
      }
      if (k0 < n) {  // ragged end of the row (n not a multiple of 64)
        const uint32_t q = k0 / 32;
        const uint32_t bits0 = n - k0;  // 1..63 header bits left
        uint32_t h_lo = __builtin_amdgcn_readlane(win, q);
        uint32_t h_hi = q + 1 < hw_n ? __builtin_amdgcn_readlane(win, q + 1) : 0u;
        if (bits0 < 32) { h_lo &= (1u << bits0) - 1u; h_hi = 0; }
        else h_hi &= (bits0 == 32) ? 0u : ((1u << (bits0 - 32)) - 1u);
        const bool valid = lane < bits0;
        const uint32_t rel =
            valid ? u + lane_keep + __umul24(cd.p, bits_below_lane(~h_lo, ~h_hi)) : 0u;
        const uint32_t x = decode_block<NR>(lds, rel, h_lo, h_hi, cd);
        if (valid) out[k0 + lane] = x;
      }
      wave_lds_sync();
    }

    if (!have_next) break;
    i = i_next;
    id = id_next;
    id_next = id_after;
    fw = fw_next;
    loc = loc_next;
    win = win_next;
  }
}

// The row pipeline shared by decode_pipe_kernel and decode_pos_pipe_kernel,
// for rows of exactly n = 64 * NCH blocks (NCH = 2, 4, 8, 16) with 16-byte
// aligned slots and output.  While row j is decoded from the wave's LDS
// window, the rest of row j+1's stream (its length known from its header,
// which arrived during row j-1) is in flight into registers, together with
// the window (first 32 words) of row j+2; so each row's dependent fetch
// overlaps the previous row's decode.  Every stream load is a buffer load
// whose range is the row's stream, and every iteration issues the same
// vector memory instructions (one window load, RV stream loads, NCH stores),
// so the waits at the top of an iteration leave the previous row's stores in
// flight.  Ids and flag words are loaded per group of 64 rows, one lane per
// row, with one clamped id per row (slot 0 stands in for a row outside the
// table, so every address is in bounds).  A wave takes rows i, i + stride,
// ...; ids past the table give zero rows.  Launches size the grid so that a
// wave has at most 64 rows: a further group restarts the pipeline.
//   stream_words(win): words of a compressed row's stream, from its window
//   decode(win, x):    the row's n words from the LDS window, x[c] = word
//                      c * 64 + lane, or with Q = 2 the 64-bit word c * 64 +
//                      lane (every lane of the wave calls it)
template <int NCH>
struct RowPipe {
  static constexpr uint32_t n = NCH * kWave;  // blocks = words of a row
  static constexpr uint32_t kWin = 32;        // window words: the header (n/32 <= 32) and more
  static constexpr int RV = (int)((n / 4 - kWin / 4 + kWave - 1) / kWave);  // units per lane
  // LDS window: every unit the loads can fill (>= n + 4 words, so a payload
  // ending in the last stream word is read with a word after it), written
  // unconditionally so that no branch separates the loads from their waits
  static constexpr uint32_t kLdsWords = kWin + RV * kWave * 4;
  static_assert(kLdsWords >= n + 4, "window too small");
};

template <int NCH, bool GATHER, int Q = 1, typename StreamWords, typename Decode>
__device__ __forceinline__ void run_row_pipeline(
    const uint32_t* __restrict__ slots, const unsigned long long* __restrict__ flags,
    const int64_t* __restrict__ ids, uint64_t n_rows, uint32_t n_out,
    uint32_t* __restrict__ dst, uint32_t* lds, uint32_t i, uint32_t stride,
    StreamWords stream_words, Decode decode) {
  using P = RowPipe<NCH>;
  constexpr uint32_t n = P::n, kWin = P::kWin;
  constexpr int RV = P::RV;
  const uint32_t lane = lane_id();
  u32x4* l4 = reinterpret_cast<u32x4*>(lds);

  // The wave's rows are i + k * stride, k = 0, 1, ..., taken in groups of up
  // to 64.  Their bookkeeping is vector work done once per group: lane k
  // loads row k's id and flag word and forms its slot address; two ballots
  // hold "in the table" and "stored compressed" for the group.  Per row the
  // scalar unit then only reads the address out of two lanes and tests a bit
  // (rows of 512 bytes are otherwise bound by the CU's one scalar unit).
  for (uint32_t g = i; g < n_out;) {
    const uint32_t K = (uint32_t)min<uint64_t>(kWave, ((uint64_t)n_out - g + stride - 1) / stride);
    const uint64_t r = (uint64_t)g + (uint64_t)lane * stride;
    const bool in = lane < K;
    const uint64_t id = in ? (GATHER ? (uint64_t)ids[r] : r) : 0ull;
    const bool ok = in && id < n_rows;
    const uint64_t idc = ok ? id : 0ull;  // slot 0 stands in for a row outside the table
    const unsigned long long fw = flags[idc >> 6];
    const uint64_t src_v = reinterpret_cast<uint64_t>(slots + idc * n);
    // bit j: row k + j of the group is in the table / stored compressed;
    // shifted down by one row per iteration, so that every test below is of
    // a fixed bit
    unsigned long long ok_m = __ballot(ok);
    unsigned long long fl_m = __ballot(ok && ((fw >> (idc & 63u)) & 1ull));

    auto src_of = [&](uint32_t k) -> const uint32_t* {
      const uint32_t kk = min(k, (uint32_t)kWave - 1u);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)src_v, kk);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(src_v >> 32), kk);
      return reinterpret_cast<const uint32_t*>(((uint64_t)hi << 32) | lo);
    };
    auto ok_of = [&](int j) { return ((uint32_t)ok_m >> j) & 1u; };
    auto fl_of = [&](int j) { return ((uint32_t)fl_m >> j) & 1u; };
    // window (first 32 words) of row k + j: a buffer load, empty past the group
    auto window = [&](int j, const uint32_t* src) -> uint32_t {
      return __builtin_amdgcn_raw_buffer_load_b32(row_rsrc(src, ok_of(j) ? kWin * 4 : 0u),
                                                  lane * 4, 0, 0);
    };
    // words of row k + j's stored form: the stream for a compressed row, the
    // whole slot for a raw one, nothing for a row outside the table
    auto stored = [&](int j, uint32_t win) -> uint32_t {
      if (!ok_of(j)) return 0u;
      if (!fl_of(j)) return n;
      return min(stream_words(win), n);
    };
    // the rest of a 4 KiB row's stream loads non-temporal (KV pages); rows of
    // 512 B to 2 KiB keep the default policy: gathers of them under Zipf ids
    // read hot rows again and again, and non-temporal loads of those made
    // the 64-bit-block dense feature and embedding gathers 1.6x slower
    constexpr int kRestPolicy = NCH >= 16 ? kLoadStream : 0;
    auto load_rest = [&](const uint32_t* src, uint32_t words, u32x4* rr) {
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, ((words + 3u) & ~3u) * 4u);
#pragma unroll
      for (int c = 0; c < RV; ++c)
        rr[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, (kWin / 4 + c * kWave + lane) * 16u, 0,
                                                      kRestPolicy);
    };

    // prologue: windows of rows 0 and 1, the stream of row 0
    const uint32_t* src0 = src_of(0);
    const uint32_t* src1 = src_of(1);
    uint32_t win0 = window(0, src0);
    uint32_t win1 = window(1, src1);
    u32x4 rest0[RV];
    load_rest(src0, stored(0, win0), rest0);
    // wait for all of it here: at the loop top the compiler merges this state
    // with the back edge's, where the previous row's stores are still pending
    asm volatile("" ::"v"(win1));
#pragma unroll
    for (int c = 0; c < RV; ++c) asm volatile("" ::"v"(rest0[c]));

    uint32_t* out = dst + (uint64_t)g * n;
    const uint64_t out_step = (uint64_t)stride * n;
    for (uint32_t k = 0;;) {
      // (1) row k's stream has arrived: stage it in the wave's LDS window
      //     (the window's lanes 32-63 are zeros that the stream units
      //     overwrite)
      lds[lane] = win0;
#pragma unroll
      for (int c = 0; c < RV; ++c) l4[kWin / 4 + c * kWave + lane] = rest0[c];
      wave_lds_sync();
      // (2) row k+1: its header gives its stream length; the rest of its
      //     stream goes in flight now
      u32x4 rest1[RV];
      load_rest(src1, stored(1, win1), rest1);
      // (3) window of row k+2
      const uint32_t* src2 = src_of(k + 2);
      const uint32_t win2 = window(2, src2);
      // (4) decode row k: exactly NCH / Q stores of Q words on every path
      using XT = std::conditional_t<Q == 2, unsigned long long, uint32_t>;
      constexpr int NX = NCH / Q;
      XT x[NX];
      if (!ok_of(0)) {
#pragma unroll
        for (int c = 0; c < NX; ++c) x[c] = 0u;
      } else if (!fl_of(0)) {
#pragma unroll
        for (int c = 0; c < NX; ++c) x[c] = reinterpret_cast<const XT*>(lds)[c * kWave + lane];
      } else {
        decode(win0, x);
      }
#pragma unroll
      for (int c = 0; c < NX; ++c)
        __builtin_nontemporal_store(x[c], reinterpret_cast<XT*>(out) + c * kWave + lane);
      __builtin_amdgcn_sched_barrier(0);
      wave_lds_sync();
      if (++k >= K) break;
      ok_m >>= 1;
      fl_m >>= 1;
      out += out_step;
      win0 = win1;
      for (int c = 0; c < RV; ++c) rest0[c] = rest1[c];
      src1 = src2;
      win1 = win2;
    }
    if ((uint64_t)g + (uint64_t)kWave * stride >= n_out) break;
    g += kWave * stride;
  }
}

// The same pipeline fetching each row's whole slot (S = 4n bytes) in one
// step instead of a window and then the rest of the stream: for rows of 512
// bytes to 2 KiB whose stored form is most of the slot (ratios near 1.1) the
// few extra bytes cost less than the dependent second fetch and the stream
// length it needs.  While row j is decoded, the slots of rows j+1 and j+2
// are in flight (FV 16-byte loads per lane each).  Every iteration issues the
// same vector memory instructions (FV loads, NCH stores), so the wait at the
// top of an iteration leaves the next row's loads and this row's stores in
// flight.  Same bookkeeping and id rules as run_row_pipeline.
//   decode(hdr, x): the row's n words from the LDS copy of its slot, x[c] =
//                   word c * 64 + lane; hdr holds header word q in lane q
template <int NCH, bool GATHER, int Q = 1, typename Decode>
__device__ __forceinline__ void run_slot_pipeline(
    const uint32_t* __restrict__ slots, const unsigned long long* __restrict__ flags,
    const int64_t* __restrict__ ids, uint64_t n_rows, uint32_t n_out,
    uint32_t* __restrict__ dst, uint32_t* lds, uint32_t i, uint32_t stride, Decode decode) {
  constexpr uint32_t n = NCH * kWave;
  constexpr int FV = NCH >= 4 ? NCH / 4 : 1;  // 16-byte loads per lane for a slot
  const uint32_t lane = lane_id();
  u32x4* l4 = reinterpret_cast<u32x4*>(lds);
  for (uint32_t g = i; g < n_out;) {
    const uint32_t K = (uint32_t)min<uint64_t>(kWave, ((uint64_t)n_out - g + stride - 1) / stride);
    const uint64_t r = (uint64_t)g + (uint64_t)lane * stride;
    const bool in = lane < K;
    const uint64_t id = in ? (GATHER ? (uint64_t)ids[r] : r) : 0ull;
    const bool ok = in && id < n_rows;
    const uint64_t idc = ok ? id : 0ull;
    const unsigned long long fw = flags[idc >> 6];
    const uint64_t src_v = reinterpret_cast<uint64_t>(slots + idc * n);
    unsigned long long ok_m = __ballot(ok);
    unsigned long long fl_m = __ballot(ok && ((fw >> (idc & 63u)) & 1ull));
    auto src_of = [&](uint32_t k) -> const uint32_t* {
      const uint32_t kk = min(k, (uint32_t)kWave - 1u);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)src_v, kk);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(src_v >> 32), kk);
      return reinterpret_cast<const uint32_t*>(((uint64_t)hi << 32) | lo);
    };
    auto ok_of = [&](int j) { return ((uint32_t)ok_m >> j) & 1u; };
    auto fl_of = [&](int j) { return ((uint32_t)fl_m >> j) & 1u; };
    // the whole slot of row k + j (nothing past the group)
    auto load_slot = [&](int j, const uint32_t* src, u32x4* v) {
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, ok_of(j) ? n * 4u : 0u);
#pragma unroll
      for (int c = 0; c < FV; ++c)
        v[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c * kWave + lane) * 16u, 0, 0);
    };
    uint32_t* out = dst + (uint64_t)g * n;
    const uint64_t out_step = (uint64_t)stride * n;
    uint32_t k = 0;
    // One row: its slot `cur` has arrived; the slot of row k+2 goes into
    // `nxt`.  The loop below is unrolled three times so that the three slot
    // buffers change roles without register copies (a copy of a buffer whose
    // load is in flight would wait for that load), and it has no exit inside
    // a round (an exit block shared with the back edge would make the
    // compiler's wait at the loop top cover the latest load); the last K % 3
    // rows follow the loop.
    auto row = [&](u32x4 (&cur)[FV], u32x4 (&nxt)[FV]) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < FV; ++c) l4[c * kWave + lane] = cur[c];
      wave_lds_sync();
      load_slot(2, src_of(k + 2), nxt);
      // NCH / Q words of Q * 32 bits per lane (Q = 2: 64-bit blocks)
      using XT = std::conditional_t<Q == 2, unsigned long long, uint32_t>;
      constexpr int NX = NCH / Q;
      XT x[NX];
      if (!ok_of(0)) {
#pragma unroll
        for (int c = 0; c < NX; ++c) x[c] = 0u;
      } else if (!fl_of(0)) {
#pragma unroll
        for (int c = 0; c < NX; ++c) x[c] = reinterpret_cast<const XT*>(lds)[c * kWave + lane];
      } else {
        decode(lds[lane], x);
      }
#pragma unroll
      for (int c = 0; c < NX; ++c)
        __builtin_nontemporal_store(x[c], reinterpret_cast<XT*>(out) + c * kWave + lane);
      __builtin_amdgcn_sched_barrier(0);
      wave_lds_sync();
      ++k;
      ok_m >>= 1;
      fl_m >>= 1;
      out += out_step;
    };
    u32x4 sa[FV], sb[FV], sc[FV];
    load_slot(0, src_of(0), sa);
    load_slot(1, src_of(1), sb);
    // wait for both here: at the loop top the compiler merges this state
    // with the back edge's, where the last rows' stores are pending
#pragma unroll
    for (int c = 0; c < FV; ++c) asm volatile("" ::"v"(sa[c]), "v"(sb[c]));
    for (uint32_t rounds = K / 3; rounds; --rounds) {
      row(sa, sc);
      row(sb, sa);
      row(sc, sb);
    }
    if (K % 3 >= 1) row(sa, sc);
    if (K % 3 == 2) row(sb, sa);
    if ((uint64_t)g + (uint64_t)kWave * stride >= n_out) break;
    g += kWave * stride;
  }
}

// The row pipeline of a kernel: whole slots (SLOT) or window + rest.
template <int NCH, bool GATHER, bool SLOT, int Q = 1, typename StreamWords, typename Decode>
__device__ __forceinline__ void row_pipeline(
    const uint32_t* __restrict__ slots, const unsigned long long* __restrict__ flags,
    const int64_t* __restrict__ ids, uint64_t n_rows, uint32_t n_out,
    uint32_t* __restrict__ dst, uint32_t* lds, uint32_t i, uint32_t stride,
    StreamWords stream_words, Decode decode) {
  if constexpr (SLOT)
    run_slot_pipeline<NCH, GATHER, Q>(slots, flags, ids, n_rows, n_out, dst, lds, i, stride,
                                      decode);
  else
    run_row_pipeline<NCH, GATHER, Q>(slots, flags, ids, n_rows, n_out, dst, lds, i, stride,
                                     stream_words, decode);
}

// [IBP] Decompression of rows of 64 * NCH blocks with one global Mask/Bitval
// (p < 32): one of the row pipelines above (SLOT: whole slots).  A compressed row's stream length is
// n + 32 n - p m bits (m = its header popcount); a payload's bit offset is
// u + 32 lane - p * (stripped blocks of the chunk below the lane).
template <int MODE, int NR, int NCH, bool SLOT = false>
__global__ __launch_bounds__(kBlockThreads) void decode_pipe_kernel(
    Codec cd, const uint32_t* __restrict__ slots, const unsigned long long* __restrict__ flags,
    const int64_t* __restrict__ ids, uint64_t n_rows, uint32_t n_out,
    uint32_t* __restrict__ dst) {
  using P = RowPipe<NCH>;
  constexpr uint32_t n = P::n;
  __shared__ __attribute__((aligned(16)))
  uint32_t lds_all[kWavesPerBlock][SLOT ? (NCH >= 4 ? n : 256u) + 4u : P::kLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint32_t stride = gridDim.x * kWavesPerBlock;
  const uint32_t i = blockIdx.x * kWavesPerBlock + wave;
  if (i >= n_out) return;
  const int negp = -(int)cd.p;
  const uint32_t l32 = 32u * lane;
  auto stream_words = [&](uint32_t win) -> uint32_t {
    const uint32_t m = wave_sum(__popc(lane < n / 32 ? win : 0u));
    return (n + 32u * n - cd.p * m + 31u) >> 5;
  };
  auto decode = [&](uint32_t win, uint32_t* x) {
    uint32_t u = n;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
      const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
      const uint32_t rel = (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + (u + l32);
      x[c] = decode_block<NR>(lds, rel, h_lo, h_hi, cd);
      u += 32u * kWave - cd.p * (uint32_t)__popcll(((unsigned long long)h_hi << 32) | h_lo);
    }
  };
  row_pipeline<NCH, MODE == kModeGather, SLOT>(slots, flags, ids, n_rows, n_out, dst, lds, i,
                                               stride, stream_words, decode);
}

// ---------------------------------------------------- other block widths --
//
// Blocks of 16 or 64 bits ([IBP] Compression cuts a tensor into blocks and
// leaves their size open: 16 bits is one fp16/bf16 element, 64 bits one fp64
// element or four half elements).  The scheme is the one above: one block
// per lane, a 64-block chunk per wave step whose 64 participation bits are
// one header word, payload offsets n + W*k - p*(stripped blocks before k) by
// v_mbcnt.  A payload has W - p or W bits; a 64-bit one is read from three
// LDS words with two funnel shifts.  Rows are whole 32-bit words (W = 16:
// an even number of blocks; W = 64: rows and buffers 8-byte aligned).

template <typename T>
struct WideCodec {
  static constexpr uint32_t W = 8 * sizeof(T);
  T mask;
  T bitval;
  uint32_t p;      // invariant bits
  uint32_t n;      // blocks per row
  uint32_t nw;     // 32-bit words per row
  uint32_t nruns;  // runs of ~mask
  uint32_t pad;    // compression: stored rows padded to 64-byte units (device slots)
  uint32_t shift[W / 2];
  T place[W / 2];
};

// Extract / deposit by the runs of ~mask; NR >= 0 is the run count known at
// compile time (unrolled, run tables in scalar registers), NR < 0 any count.
template <typename T, int NR>
__device__ __forceinline__ T extract_wide(T x, const WideCodec<T>& cd) {
  T v = 0;
  if constexpr (NR >= 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) v |= (T)((x & cd.place[j]) >> cd.shift[j]);
  } else {
    for (uint32_t j = 0; j < cd.nruns; ++j) v |= (T)((x & cd.place[j]) >> cd.shift[j]);
  }
  return v;
}

template <typename T, int NR>
__device__ __forceinline__ T deposit_wide(T v, const WideCodec<T>& cd) {
  T x = cd.bitval;
  if constexpr (NR >= 0) {
#pragma unroll
    for (int j = 0; j < NR; ++j) x |= (T)((T)(v << cd.shift[j]) & cd.place[j]);
  } else {
    for (uint32_t j = 0; j < cd.nruns; ++j) x |= (T)((T)(v << cd.shift[j]) & cd.place[j]);
  }
  return x;
}

// The W bits of the stream at bit `rel` of the LDS window (bits past the
// payload's length come from the next payload and are never used).
template <typename T>
__device__ __forceinline__ T lds_payload(const uint32_t* lds, uint32_t rel) {
  const uint32_t wi = rel >> 5, s = rel & 31u;
  const uint32_t lo = __builtin_amdgcn_alignbit(lds[wi + 1], lds[wi], s);
  if constexpr (sizeof(T) == 8) {
    const uint32_t hi = __builtin_amdgcn_alignbit(lds[wi + 2], lds[wi + 1], s);
    return ((uint64_t)hi << 32) | lo;
  } else {
    return (T)lo;
  }
}

// [IBP] Compression for W = 16 / 64, one workgroup per row (the stream is
// assembled in LDS as in compress_kernel; in place is safe the same way).
template <typename T, int NR, uint32_t MAXW>
__global__ __launch_bounds__(kBlockThreads) void compress_wide_kernel(
    WideCodec<T> cd, uint64_t n_rows, const uint32_t* src, uint32_t* slots,
    unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits) {
  constexpr uint32_t W = WideCodec<T>::W;
  __shared__ uint32_t buf[MAXW + 4];
  __shared__ uint32_t chunk_pre[(MAXW * 32 / W + kWave - 1) / kWave];
  __shared__ uint32_t total_m;
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t n = cd.n, nw = cd.nw;
  const uint32_t nchunks = (n + kWave - 1) / kWave;

  for (uint64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    const T* x_row = reinterpret_cast<const T*>(src + row * nw);
    uint32_t* s_row = slots + row * nw;
    for (uint32_t j = threadIdx.x; j < nw + 4; j += kBlockThreads) buf[j] = 0;
    __syncthreads();
    for (uint32_t c = wave; c < nchunks; c += kWavesPerBlock) {
      const uint32_t k = c * kWave + lane;
      const bool valid = k < n;
      const T x = valid ? x_row[k] : (T)0;
      const unsigned long long h = __ballot(valid && (T)(x & cd.mask) == cd.bitval);
      if (lane == 0) {
        chunk_pre[c] = (uint32_t)__popcll(h);
        buf[2 * c] = (uint32_t)h;
        if (2 * c + 1 < (n + 31) / 32) buf[2 * c + 1] = (uint32_t)(h >> 32);
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t carry = 0;
      for (uint32_t b0 = 0; b0 < nchunks; b0 += kWave) {
        const uint32_t c = b0 + lane;
        const uint32_t v = c < nchunks ? chunk_pre[c] : 0u;
        const uint32_t inc = wave_inclusive_scan(v, lane);
        if (c < nchunks) chunk_pre[c] = carry + inc - v;
        carry += __shfl(inc, kWave - 1, kWave);
      }
      if (lane == 0) total_m = carry;
    }
    __syncthreads();
    const uint32_t m = total_m;
    const uint32_t c_bits = n + W * n - cd.p * m;
    const bool flag = c_bits < W * n;
    if (!flag) {
      const uint32_t* xr = src + row * nw;
      for (uint32_t j = threadIdx.x; j < nw; j += kBlockThreads) s_row[j] = xr[j];
    } else {
      for (uint32_t c = wave; c < nchunks; c += kWavesPerBlock) {
        const uint32_t k = c * kWave + lane;
        const bool valid = k < n;
        const T x = valid ? x_row[k] : (T)0;
        const bool match = valid && (T)(x & cd.mask) == cd.bitval;
        const unsigned long long h = __ballot(match);
        const uint32_t pre = chunk_pre[c] + bits_below_lane((uint32_t)h, (uint32_t)(h >> 32));
        if (valid) {
          const uint32_t off = n + W * k - cd.p * pre;
          const uint32_t len = match ? W - cd.p : W;
          const uint64_t pay = match ? (uint64_t)extract_wide<T, NR>(x, cd) : (uint64_t)x;
          if (len) {
            const uint32_t sh = off & 31u, wi = off >> 5;
            const uint64_t lo = pay << sh;  // bits [0, 64) of the placed payload
            atomicOr(&buf[wi], (uint32_t)lo);
            if (sh + len > 32u) atomicOr(&buf[wi + 1], (uint32_t)(lo >> 32));
            if (sh + len > 64u) atomicOr(&buf[wi + 2], (uint32_t)(pay >> (64u - sh)));
          }
        }
      }
      __syncthreads();
      const uint32_t words = (c_bits + 31u) >> 5;
      for (uint32_t j = threadIdx.x; j < words; j += kBlockThreads) __builtin_nontemporal_store(buf[j], &s_row[j]);
    }
    if (threadIdx.x == 0) {
      put_flag_bits(flags, row, 1u, flag ? 1ull : 0ull, n_rows);
      if (row_bits) row_bits[row] = c_bits;
    }
    // the LDS stream is reused only by a next row; after the last one the
    // workgroup ends without waiting for its stores (a barrier would)
    if (row + gridDim.x < n_rows) __syncthreads();
  }
}

// [IBP] Compression with 16-bit blocks of rows of exactly 128 * NWL blocks
// (64 * NWL words), one wave per row with the row in registers: lane l holds
// word 64 t + l, blocks 2 (64 t + l) and 2 (64 t + l) + 1 of the 128-block
// step t.  Two ballots per step (first / second block of the pair matches)
// count the stripped blocks and, through v_mbcnt, give each pair's offset;
// the step's four header words are the pairs' two bits ORed across each row
// of 16 lanes (DPP).  One extract over the packed pair, with the run masks
// repeated in both halves, strips both blocks (run j moves bits down by
// shift_j, and a half's bits never leave it); the pair's payloads, joined,
// take at most 32 bits, ORed into the wave's LDS stream.  In place is safe:
// the row is read whole before the first store.
template <int NR, int NWL>
__global__ __launch_bounds__(kBlockThreads) void compress_pair_rows_kernel(
    WideCodec<uint16_t> cd, uint64_t n_rows, const uint32_t* src, uint32_t* slots,
    unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits) {
  constexpr uint32_t nw = (uint32_t)NWL * kWave;  // words of a row
  constexpr uint32_t n = 2u * nw;                 // 16-bit blocks of a row
  __shared__ uint32_t lds_all[kWavesPerBlock][nw + 4];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds_all[wave];
  const uint32_t m2 = (uint32_t)cd.mask * 0x10001u, b2 = (uint32_t)cd.bitval * 0x10001u;
  const uint32_t sh = 2u * (lane & 15u);
  auto extract2 = [&](uint32_t y) -> uint32_t {
    uint32_t v = 0;
    if constexpr (NR >= 0) {
#pragma unroll
      for (int j = 0; j < NR; ++j) v |= (y & ((uint32_t)cd.place[j] * 0x10001u)) >> cd.shift[j];
    } else {
      for (uint32_t j = 0; j < cd.nruns; ++j)
        v |= (y & ((uint32_t)cd.place[j] * 0x10001u)) >> cd.shift[j];
    }
    return v;
  };
  compress_row_range(n_rows, wave, kWavesPerBlock, 16u * n, flags, row_bits, [&](uint64_t row) {
    const __amdgpu_buffer_rsrc_t in = row_rsrc(src + row * nw, nw * 4u);
    uint32_t x[NWL];
    unsigned long long e[NWL], o[NWL];
#pragma unroll
    for (int t = 0; t < NWL; ++t)
      x[t] = __builtin_amdgcn_raw_buffer_load_b32(in, (t * kWave + lane) * 4u, 0, kRowLoad);
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < NWL; ++t) {
      const uint32_t d = (x[t] & m2) ^ b2;
      e[t] = __ballot((d & 0xFFFFu) == 0u);
      o[t] = __ballot((d >> 16) == 0u);
      m += (uint32_t)(__popcll(e[t]) + __popcll(o[t]));
    }
    const uint32_t c_bits = n + 16u * n - cd.p * m;
    const bool flag = c_bits < 16u * n;
    uint32_t nwc = nw;
    if (flag) {
      nwc = store_words(slots + row * nw, (c_bits + 31u) >> 5, nw, cd.pad);
      for (uint32_t j = n / 32 + lane; j < nwc + 1; j += kWave) buf[j] = 0u;
#pragma unroll
      for (int t = 0; t < NWL; ++t) {
        uint32_t v = (__builtin_amdgcn_inverse_ballot_w64(e[t]) ? 1u : 0u) |
                     (__builtin_amdgcn_inverse_ballot_w64(o[t]) ? 2u : 0u);
        v <<= sh;
        v |= __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false);  // row_shr:1
        v |= __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false);  // row_shr:2
        v |= __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);  // row_shr:4
        v |= __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false);  // row_shr:8
        if ((lane & 15u) == 15u) buf[4 * t + (lane >> 4)] = v;
      }
      wave_lds_sync();
      uint32_t carry = 0;
#pragma unroll
      for (int t = 0; t < NWL; ++t) {
        const bool s0 = __builtin_amdgcn_inverse_ballot_w64(e[t]);
        const bool s1 = __builtin_amdgcn_inverse_ballot_w64(o[t]);
        const uint32_t below = bits_below_lane_acc(
            (uint32_t)o[t], (uint32_t)(o[t] >> 32),
            bits_below_lane((uint32_t)e[t], (uint32_t)(e[t] >> 32)));
        const uint32_t off =
            n + 16u * (2u * (t * kWave + lane)) - __umul24(cd.p, carry + below);
        const uint32_t l0 = s0 ? 16u - cd.p : 16u;
        const uint32_t l1 = s1 ? 16u - cd.p : 16u;
        const uint32_t ext = extract2(x[t]);
        const uint32_t pay0 = (s0 ? ext : x[t]) & 0xFFFFu;
        const uint32_t pay1 = (s1 ? ext : x[t]) >> 16;
        const uint32_t pay = pay0 | (pay1 << l0);
        const uint32_t len = l0 + l1;
        if (len) {
          const uint32_t sw = off & 31u, wi = off >> 5;
          atomicOr(&buf[wi], pay << sw);
          if (sw + len > 32u) atomicOr(&buf[wi + 1], pay >> (32u - sw));
        }
        carry += (uint32_t)(__popcll(e[t]) + __popcll(o[t]));
      }
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < NWL; ++t) x[t] = t * kWave < nwc ? buf[t * kWave + lane] : 0u;
    }
    const __amdgpu_buffer_rsrc_t out = row_rsrc(slots + row * nw, nwc * 4u);
#pragma unroll
    for (int t = 0; t < NWL; ++t)
      __builtin_amdgcn_raw_buffer_store_b32(x[t], out, (t * kWave + lane) * 4u, 0, kRowStore);
    wave_lds_sync();
    return c_bits;
  });
}

// [IBP] Compression with 16-bit blocks of rows of exactly 256 * CPW words
// (512 * CPW blocks; the 8 and 28 KiB rows of bf16 weight matrices), one
// workgroup per row.  Each wave holds a quarter of the row in registers, one
// word (two blocks) per lane per chunk, as in compress_pair_rows_kernel: the
// pairs' two header bits are ORed into the chunk's four header words across
// each row of 16 lanes, the waves' match totals meet in LDS to give each wave
// its carry, and the joined payloads of a pair are ORed into the
// workgroup's LDS stream, which is then written with coalesced stores (a raw
// row straight from the registers).  Three barriers per row.  As in
// compress_wg_kernel, a workgroup takes a contiguous range of `per_wg` rows
// (at most 64), loads its next row while it encodes one, writes the range's
// flag bits once at its end (whole bytes when per_wg is a multiple of 8) and
// takes up to kCompressBatchMax tensors of one row length per launch.  In
// place is safe: every wave has read its part of the row before the first
// barrier, and the row loaded ahead is another row.
template <int NR, int CPW>
__global__ __launch_bounds__(kBlockThreads) void compress_pair_wg_kernel(
    WideCodec<uint16_t> cd, CompressBatch batch, uint32_t per_wg) {
  uint32_t t = 0;
  while (blockIdx.x >= batch.wg_end[t]) ++t;
  const CompressTensor& ct = batch.t[t];
  const uint64_t n_rows = ct.n_rows;
  const uint32_t* src = ct.src;
  uint32_t* slots = ct.slots;
  unsigned long long* flags = ct.flags;
  uint32_t* row_bits = ct.row_bits;
  const uint32_t wg = blockIdx.x - (t ? batch.wg_end[t - 1] : 0u);  // within the tensor
  constexpr uint32_t nw = (uint32_t)CPW * kWave * kWavesPerBlock;  // words of a row
  constexpr uint32_t n = 2u * nw;                                   // blocks of a row
  __shared__ uint32_t buf[nw + 4];
  __shared__ uint32_t wtot[kWavesPerBlock];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t c0 = wave * CPW;  // the wave's first chunk of 64 words
  const uint32_t lane_byte = (c0 * kWave + lane) * 4u;
  const uint32_t m2 = (uint32_t)cd.mask * 0x10001u, b2 = (uint32_t)cd.bitval * 0x10001u;
  const uint32_t sh = 2u * (lane & 15u);
  // a run's kept bits at their payload position, in both halves of a word:
  // extract = OR of (y >> shift) & kept2, a shift and an and-or per run
  constexpr int NK = NR > 0 ? NR : 1;
  uint32_t kept2[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j)
    kept2[j] = NR > 0 ? ((uint32_t)cd.place[j] >> cd.shift[j]) * 0x10001u : 0u;
  auto extract2 = [&](uint32_t y) -> uint32_t {
    uint32_t v = 0;
    if constexpr (NR >= 0) {
#pragma unroll
      for (int j = 0; j < NR; ++j) v |= (y >> cd.shift[j]) & kept2[j];
    } else {
      for (uint32_t j = 0; j < cd.nruns; ++j)
        v |= (y & ((uint32_t)cd.place[j] * 0x10001u)) >> cd.shift[j];
    }
    return v;
  };
  const uint64_t r0 = (uint64_t)wg * per_wg;
  const uint64_t r1 = min(n_rows, r0 + per_wg);
  // a row past the range loads as zeros (empty range), never out of bounds
  auto load = [&](uint32_t (&v)[CPW], uint64_t r) {
    const __amdgpu_buffer_rsrc_t in =
        row_rsrc(src + (r < r1 ? r : r0) * nw, r < r1 ? nw * 4u : 0u);
    uint32_t lb = lane_byte;  // opaque: the chunks' offsets are immediates on it
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      v[c] = __builtin_amdgcn_raw_buffer_load_b32(in, lb + c * kWave * 4u, 0, kRowLoad);
  };
  uint32_t x[CPW];
  load(x, r0);
  unsigned long long fl = 0;  // bit j: row r0 + j is stored compressed
  for (uint64_t row = r0; row < r1; ++row) {
    uint32_t* s_row = slots + row * nw;
    uint32_t y[CPW];  // the next row, in flight
    load(y, row + 1);
    // the payload part of the stream starts zeroed; header words are whole
    for (uint32_t j = n / 32 + threadIdx.x; j < nw + 4; j += kBlockThreads) buf[j] = 0u;
    uint32_t mw = 0;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t d = (x[c] & m2) ^ b2;
      const unsigned long long e = __ballot((d & 0xFFFFu) == 0u);
      const unsigned long long o = __ballot((d >> 16) == 0u);
      mw += (uint32_t)(__popcll(e) + __popcll(o));
      uint32_t v = (__builtin_amdgcn_inverse_ballot_w64(e) ? 1u : 0u) |
                   (__builtin_amdgcn_inverse_ballot_w64(o) ? 2u : 0u);
      v <<= sh;
      v |= __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false);  // row_shr:1
      v |= __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false);  // row_shr:2
      v |= __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);  // row_shr:4
      v |= __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false);  // row_shr:8
      if ((lane & 15u) == 15u) buf[4u * (c0 + c) + (lane >> 4)] = v;
    }
    if (lane == 0) wtot[wave] = mw;
    __syncthreads();
    uint32_t carry = 0, m = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const uint32_t t = wtot[w];
      carry += (uint32_t)w < wave ? t : 0u;
      m += t;
    }
    const uint32_t c_bits = n + 16u * n - cd.p * m;
    const bool flag = c_bits < 16u * n;
    fl |= (unsigned long long)flag << (row - r0);
    if (flag) {
      // the lane's first pair offset less the carry, opaque (folded into CPW
      // loop-invariant chunk bases it would hold as many registers)
      uint32_t ob = n + 8u * lane_byte;
      asm volatile("" : "+v"(ob));
      const int negp = -(int)cd.p;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        // the match tests again (cheaper than turning kept ballots back
        // into lane masks)
        asm volatile("" : "+v"(x[c]));
        const uint32_t d = (x[c] & m2) ^ b2;
        const bool s0 = (d & 0xFFFFu) == 0u;
        const bool s1 = (d >> 16) == 0u;
        const unsigned long long e = __ballot(s0);
        const unsigned long long o = __ballot(s1);
        const uint32_t below = bits_below_lane_acc(
            (uint32_t)o, (uint32_t)(o >> 32), bits_below_lane((uint32_t)e, (uint32_t)(e >> 32)));
        uint32_t t = (uint32_t)(c * kWave * 32) - cd.p * carry;
        asm volatile("" : "+s"(t));
        const uint32_t off = (uint32_t)mul_i24((int)below, negp) + ob + t;
        const uint32_t l0 = s0 ? 16u - cd.p : 16u;
        const uint32_t ext = extract2(x[c]);
        const uint32_t pay0 = (s0 ? ext : x[c]) & 0xFFFFu;
        const uint32_t pay1 = (s1 ? ext : x[c]) >> 16;
        const uint32_t pay = pay0 | (pay1 << l0);
        // the pair's bits in its first stream word and the next (zero when
        // they end in the first).  With p = 16 a pair of stripped blocks has
        // no payload and takes no part (many empty payloads at one offset
        // would all hit one LDS word); otherwise no branch.
        const unsigned long long w2 = (unsigned long long)pay << (off & 31u);
        if (NR != 0 || !(s0 && s1)) {
          atomicOr(&buf[off >> 5], (uint32_t)w2);
          atomicOr(&buf[(off >> 5) + 1u], (uint32_t)(w2 >> 32));
        }
        carry += (uint32_t)(__popcll(e) + __popcll(o));
      }
    }
    __syncthreads();
    if (!flag) {
      const __amdgpu_buffer_rsrc_t out = row_rsrc(s_row, nw * 4u);
      uint32_t lb = lane_byte;
      asm volatile("" : "+v"(lb));
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        __builtin_amdgcn_raw_buffer_store_b32(x[c], out, lb + c * kWave * 4u, 0, kRowStore);
    } else {
      const uint32_t nwc = store_words(s_row, (c_bits + 31u) >> 5, nw, ct.pad);
      uint32_t j0 = 0;
      if ((reinterpret_cast<uintptr_t>(s_row) & 15u) == 0) {  // whole 16-byte units
        const u32x4* b4 = reinterpret_cast<const u32x4*>(buf);
        u32x4* o4 = reinterpret_cast<u32x4*>(s_row);
        for (uint32_t j = threadIdx.x; j < nwc / 4; j += kBlockThreads) __builtin_nontemporal_store(b4[j], &o4[j]);
        j0 = nwc & ~3u;
      }
      for (uint32_t j = j0 + threadIdx.x; j < nwc; j += kBlockThreads) __builtin_nontemporal_store(buf[j], &s_row[j]);
    }
    if (threadIdx.x == 0 && row_bits) row_bits[row] = c_bits;
#pragma unroll
    for (int c = 0; c < CPW; ++c) x[c] = y[c];
    // the LDS stream is reused only by a next row; after the last one the
    // workgroup ends without waiting for its stores (a barrier would)
    if (row + 1 < r1) __syncthreads();
  }
  if (wave == 0 && r0 < r1) {
    const uint32_t k = (uint32_t)(r1 - r0);
    if (per_wg % 8u == 0)
      put_flag_bytes(flags, r0, k, fl, n_rows, lane);
    else if (lane == 0)
      put_flag_bits(flags, r0, k, fl, n_rows);
  }
}

// [IBP] Compression with 64-bit blocks of rows of exactly 64 * NCH blocks
// (512 bytes to 4 KiB), one wave per row with the row in registers (lane l
// holds block 64 c + l of chunk c): each chunk's match ballot is its header
// word pair, the chunk prefixes are a scalar running sum, and a payload of up
// to 64 bits is ORed into the wave's LDS stream in up to three words.  In
// place is safe: the row is read whole before the first store.
template <int NR, int NCH>
__global__ __launch_bounds__(kBlockThreads) void compress_w64_rows_kernel(
    WideCodec<uint64_t> cd, uint64_t n_rows, const uint32_t* src, uint32_t* slots,
    unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits) {
  constexpr uint32_t nb = (uint32_t)NCH * kWave;  // blocks of a row
  constexpr uint32_t nw = 2u * nb;                // words of a row
  __shared__ uint32_t lds_all[kWavesPerBlock][nw + 4];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds_all[wave];
  compress_row_range(n_rows, wave, kWavesPerBlock, 64u * nb, flags, row_bits, [&](uint64_t row) {
    const uint64_t* x_row = reinterpret_cast<const uint64_t*>(src + row * nw);
    uint64_t* s_row64 = reinterpret_cast<uint64_t*>(slots + row * nw);
    uint64_t x[NCH];
    unsigned long long h[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) x[c] = __builtin_nontemporal_load(&x_row[c * kWave + lane]);
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      h[c] = __ballot((x[c] & cd.mask) == cd.bitval);
      m += (uint32_t)__popcll(h[c]);
    }
    const uint32_t c_bits = nb + 64u * nb - cd.p * m;
    const bool flag = c_bits < 64u * nb;
    if (!flag) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) __builtin_nontemporal_store(x[c], &s_row64[c * kWave + lane]);
    } else {
      const uint32_t nwc = store_words(slots + row * nw, (c_bits + 31u) >> 5, nw, cd.pad);
      for (uint32_t j = nb / 32 + lane; j < nwc + 2; j += kWave) buf[j] = 0u;
      if (lane < 2 * NCH) {  // header word q = half (q & 1) of chunk q / 2's ballot
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          if (lane == 2u * c) w = (uint32_t)h[c];
          if (lane == 2u * c + 1) w = (uint32_t)(h[c] >> 32);
        }
        buf[lane] = w;
      }
      wave_lds_sync();
      uint32_t carry = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t lo = (uint32_t)h[c], hi = (uint32_t)(h[c] >> 32);
        const bool match = __builtin_amdgcn_inverse_ballot_w64(h[c]);
        const uint32_t off =
            nb + 64u * (c * kWave + lane) - __umul24(cd.p, carry + bits_below_lane(lo, hi));
        const uint32_t len = match ? 64u - cd.p : 64u;
        const uint64_t pay = match ? extract_wide<uint64_t, NR>(x[c], cd) : x[c];
        if (len) {
          const uint32_t sh = off & 31u, wi = off >> 5;
          const uint64_t placed = pay << sh;  // bits [0, 64) of the placed payload
          atomicOr(&buf[wi], (uint32_t)placed);
          if (sh + len > 32u) atomicOr(&buf[wi + 1], (uint32_t)(placed >> 32));
          if (sh + len > 64u) atomicOr(&buf[wi + 2], (uint32_t)(pay >> (64u - sh)));
        }
        carry += (uint32_t)__popcll(h[c]);
      }
      wave_lds_sync();
      uint32_t v[2 * NCH];
#pragma unroll
      for (int t = 0; t < 2 * NCH; ++t) v[t] = t * kWave < nwc ? buf[t * kWave + lane] : 0u;
      const __amdgpu_buffer_rsrc_t out = row_rsrc(slots + row * nw, nwc * 4u);
#pragma unroll
      for (int t = 0; t < 2 * NCH; ++t)
        __builtin_amdgcn_raw_buffer_store_b32(v[t], out, (t * kWave + lane) * 4u, 0, kRowStore);
      wave_lds_sync();
    }
    return c_bits;
  });
}

// [IBP] Compression with 64-bit blocks of the long weight rows (1024, 2048,
// 3584 or 4096 blocks: 8, 16, 28 and 32 KiB), a workgroup of four waves per
// row, the scheme of compress_wg_kernel: each wave holds CPW chunks of the
// row in registers (one block per lane each), so the row is read once; the
// chunk ballots are the header word pairs (placed in their lanes with lane
// writes); the waves' match totals meet in LDS and give each wave its carry;
// a payload of up to 64 bits is ORed into the workgroup's LDS stream in up to
// three words, and the stream is written with coalesced stores (a raw row
// straight from the registers).  A workgroup takes a contiguous range of
// `per_wg` rows with the next row in flight and writes the range's flag bits
// once (whole bytes when per_wg is a multiple of 8).  In place is safe as in
// compress_wg_kernel.  One launch takes up to kCompressBatchMax tensors of
// one row length.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NR, int CPW>
__global__ __launch_bounds__(kBlockThreads) void compress_w64_wg_kernel(
    WideCodec<uint64_t> cd, CompressBatch batch, uint32_t per_wg) {
  uint32_t t = 0;
  while (blockIdx.x >= batch.wg_end[t]) ++t;
  const CompressTensor& ct = batch.t[t];
  const uint64_t n_rows = ct.n_rows;
  const uint32_t* src = ct.src;
  uint32_t* slots = ct.slots;
  unsigned long long* flags = ct.flags;
  uint32_t* row_bits = ct.row_bits;
  const uint32_t wg = blockIdx.x - (t ? batch.wg_end[t - 1] : 0u);  // within the tensor
  constexpr uint32_t nb = (uint32_t)CPW * kWave * kWavesPerBlock;  // blocks of a row
  constexpr uint32_t nw = 2u * nb;                                  // words of a row
  __shared__ uint32_t buf[nw + 4];
  __shared__ uint32_t wtot[kWavesPerBlock];  // the waves' match totals
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t c0 = wave * CPW;                        // the wave's first chunk
  const uint32_t lane_byte = (c0 * kWave + lane) * 8u;   // its first block's byte
  const int negp = -(int)cd.p;
  const uint64_t r0 = (uint64_t)wg * per_wg;
  const uint64_t r1 = min(n_rows, r0 + per_wg);
  // a row past the range loads as zeros (empty range), never out of bounds
  auto load = [&](uint64_t (&v)[CPW], uint64_t r) {
    const __amdgpu_buffer_rsrc_t in =
        row_rsrc(src + (r < r1 ? r : r0) * nw, r < r1 ? nw * 4u : 0u);
    uint32_t lb = lane_byte;  // opaque: the chunks' offsets are immediates on it
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(in, lb + c * kWave * 8u, 0, kRowLoad);
      v[c] = ((uint64_t)w.y << 32) | w.x;
    }
  };
  uint64_t x[CPW];
  load(x, r0);
  unsigned long long fl = 0;  // bit j: row r0 + j is stored compressed
  for (uint64_t row = r0; row < r1; ++row) {
    uint32_t* s_row = slots + row * nw;
    uint64_t y[CPW];  // the next row, in flight
    load(y, row + 1);
    // the payload part of the stream starts zeroed; header words are whole
    for (uint32_t j = nb / 32 + threadIdx.x; j < nw + 4; j += kBlockThreads) buf[j] = 0u;
    uint32_t mw = 0;
    uint32_t hword = 0;  // lane 2c / 2c + 1: low / high half of chunk c's ballot
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const unsigned long long h = __ballot((x[c] & cd.mask) == cd.bitval);
      mw += (uint32_t)__popcll(h);
      hword = (uint32_t)lane_write((int)(uint32_t)h, 2 * c, (int)hword);
      hword = (uint32_t)lane_write((int)(uint32_t)(h >> 32), 2 * c + 1, (int)hword);
    }
    if (lane < 2u * CPW) buf[2u * c0 + lane] = hword;
    if (lane == 0) wtot[wave] = mw;
    __syncthreads();
    uint32_t carry = 0, m = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const uint32_t tw = wtot[w];
      carry += (uint32_t)w < wave ? tw : 0u;
      m += tw;
    }
    const uint32_t c_bits = nb + 64u * nb - cd.p * m;
    const bool flag = c_bits < 64u * nb;
    fl |= (unsigned long long)flag << (row - r0);
    if (flag) {
      // the lane's first payload offset less the carry: the stream's nb
      // header bits, then 64 bits per block before it (opaque, as in
      // compress_wg_kernel)
      uint32_t ob = nb + 8u * lane_byte;
      asm volatile("" : "+v"(ob));
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const bool match = (x[c] & cd.mask) == cd.bitval;
        const unsigned long long h = __ballot(match);
        const uint32_t below = bits_below_lane((uint32_t)h, (uint32_t)(h >> 32));
        uint32_t tc = (uint32_t)(c * kWave * 64) - cd.p * carry;
        asm volatile("" : "+s"(tc));
        const uint32_t off = (uint32_t)mul_i24((int)below, negp) + ob + tc;
        const uint32_t sh = off & 31u, wi = off >> 5;
        if constexpr (NR != 0) {
          // p < 64: every block has a payload of 64 - p or 64 bits; its
          // first two stream words get their bits with no branch
          const uint64_t pay = match ? extract_wide<uint64_t, NR>(x[c], cd) : x[c];
          const uint32_t len = match ? 64u - cd.p : 64u;
          const uint64_t placed = pay << sh;
          atomicOr(&buf[wi], (uint32_t)placed);
          atomicOr(&buf[wi + 1u], (uint32_t)(placed >> 32));
          if (sh + len > 64u) atomicOr(&buf[wi + 2u], (uint32_t)(pay >> (64u - sh)));
        } else {
          // p = 64: a stripped block has no payload
          if (!match) {
            const uint64_t placed = x[c] << sh;
            atomicOr(&buf[wi], (uint32_t)placed);
            atomicOr(&buf[wi + 1u], (uint32_t)(placed >> 32));
            if (sh) atomicOr(&buf[wi + 2u], (uint32_t)(x[c] >> (64u - sh)));
          }
        }
        carry += (uint32_t)__popcll(h);
      }
    }
    __syncthreads();
    if (!flag) {
      const __amdgpu_buffer_rsrc_t out = row_rsrc(s_row, nw * 4u);
      uint32_t lb = lane_byte;
      asm volatile("" : "+v"(lb));
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{(uint32_t)x[c], (uint32_t)(x[c] >> 32)},
                                              out, lb + c * kWave * 8u, 0, kRowStore);
    } else {
      const uint32_t nwc = store_words(s_row, (c_bits + 31u) >> 5, nw, ct.pad);
      uint32_t j0 = 0;
      if ((reinterpret_cast<uintptr_t>(s_row) & 15u) == 0) {  // whole 16-byte units
        const u32x4* b4 = reinterpret_cast<const u32x4*>(buf);
        u32x4* o4 = reinterpret_cast<u32x4*>(s_row);
        for (uint32_t j = threadIdx.x; j < nwc / 4; j += kBlockThreads) __builtin_nontemporal_store(b4[j], &o4[j]);
        j0 = nwc & ~3u;
      }
      for (uint32_t j = j0 + threadIdx.x; j < nwc; j += kBlockThreads) __builtin_nontemporal_store(buf[j], &s_row[j]);
    }
    if (threadIdx.x == 0 && row_bits) row_bits[row] = c_bits;
#pragma unroll
    for (int c = 0; c < CPW; ++c) x[c] = y[c];
    // the LDS stream is reused only by a next row; after the last one the
    // workgroup ends without waiting for its stores (a barrier would)
    if (row + 1 < r1) __syncthreads();
  }
  if (wave == 0 && r0 < r1) {
    const uint32_t k = (uint32_t)(r1 - r0);
    if (per_wg % 8u == 0)
      put_flag_bytes(flags, r0, k, fl, n_rows, lane);
    else if (lane == 0)
      put_flag_bits(flags, r0, k, fl, n_rows);
  }
}

// Blocks per decode task for W = 16 / 64: a segment's stream stays within
// the LDS window of a 32-bit segment (seg * W / 32 <= kSegBlocks words).
template <typename T>
constexpr uint32_t wide_seg_blocks() {
  return kSegBlocks * 32u / (8u * (uint32_t)sizeof(T));
}

// [IBP] Decompression for W = 16 / 64 of one task: segment s (blocks
// [s * seg, min(n, (s + 1) * seg))) of output row i (rows of n blocks, slots
// of nw words), in the three row-source modes of the 32-bit kernels.
template <typename T, int MODE, int NR>
__device__ __forceinline__ void decode_wide_task(
    const WideCodec<T>& cd, uint32_t n, uint32_t nw, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    const uint32_t* __restrict__ arena, const unsigned long long* __restrict__ cache_loc,
    uint64_t n_rows, uint64_t i, uint32_t s, uint32_t seg, T* __restrict__ dst, int vec,
    uint32_t* lds, uint32_t lane) {
  constexpr uint32_t W = WideCodec<T>::W;
  const uint64_t id = MODE != kModeTable ? (uint64_t)ids[i] : i;
  T* out = dst + i * n;
  const uint32_t lo = s * seg;
  const uint32_t hi = min(n, lo + seg);
  if (MODE != kModeTable && id >= n_rows) {
    for (uint32_t j = lo + lane; j < hi; j += kWave) out[j] = (T)0;
    return;
  }
  const unsigned long long loc = MODE == kModeCached ? cache_loc[id] : 0ull;
  const unsigned long long fw = (loc & IBP_LOC_RESIDENT) ? 0ull : flags[id >> 6];
  const uint32_t* src = row_source<MODE>(slots, arena, id, nw, loc);
  const uint32_t lim = row_words<MODE>(nw, loc);
  // header words requested with the flag word (see decode_segments_kernel)
  const uint32_t hw_n = (hi - lo + 31) / 32;
  uint32_t hw = 0;
  if (lane < hw_n) hw = src[lo / 32 + lane];
  uint32_t acc = 0;
  for (uint32_t t0 = 0; t0 < lo / 32; t0 += 4 * kWave) {
    uint32_t w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = src[min(t0 + c * kWave + lane, lo / 32 - 1)];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc += t0 + c * kWave + lane < lo / 32 ? __popc(w[c]) : 0u;
  }
  if (!row_flag<MODE>(fw, id, loc)) {
    if (vec) {  // 16-byte units of the segment (lo and hi are multiples of 16 bytes)
      const uint4* a = reinterpret_cast<const uint4*>(src);
      uint4* o = reinterpret_cast<uint4*>(out);
      constexpr uint32_t per = 16 / sizeof(T);
      for (uint32_t j = lo / per + lane; j < hi / per; j += kWave) o[j] = a[j];
    } else {
      const T* a = reinterpret_cast<const T*>(src);
      for (uint32_t j = lo + lane; j < hi; j += kWave) out[j] = a[j];
    }
    return;
  }
  // stripped blocks before the segment (lo is a multiple of 64)
  const uint32_t carry = lo ? wave_sum(acc) : 0u;
  if (lane < hw_n) {
    const uint32_t valid_bits = min(32u, hi - 32u * (lo / 32 + lane));
    if (valid_bits < 32u) hw &= (1u << valid_bits) - 1u;
  }
  const uint32_t m_seg = wave_sum(__popc(hw));
  const uint32_t a = n + W * lo - cd.p * carry;
  const uint32_t b = n + W * hi - cd.p * (carry + m_seg);
  const uint32_t wb = min((b + 31u) >> 5, lim);
  const uint32_t wa = min(a >> 5, wb);
  uint32_t base = wa;
  if (vec) {  // 16-byte loads from the 16-byte unit holding word wa
    base = wa & ~3u;
    stage_window<5, MODE != kModeCached>(reinterpret_cast<const u32x4*>(src + base),
                                         reinterpret_cast<u32x4*>(lds), (wb - base + 3u) / 4u,
                                         lane);
  } else {
    stage_window<4, MODE != kModeCached>(src + wa, lds, wb - wa, lane);
  }
  wave_lds_sync();
  uint32_t u = a - 32u * base;
  const int negp = -(int)cd.p;
  // a whole segment (the decode launch cuts rows into segments of 2048
  // blocks for W = 16 and 512 for W = 64) unrolled, anything shorter step
  // by step
  constexpr uint32_t kFull = wide_seg_blocks<T>();
  if constexpr (sizeof(T) == 2) {
    // Two blocks per lane: lane l restores blocks k0 + 2l and k0 + 2l + 1
    // of a 128-block step and stores them as one word.  Their header bits
    // are bits 2(l mod 16) and 2(l mod 16) + 1 of header word q + l/16;
    // two ballots (first / second block of a pair stripped) give the
    // stripped blocks before the pair through v_mbcnt.  Both payloads lie
    // in the 32 stream bits at the pair's offset (16 - p or 16 bits each),
    // and one deposit over the packed pair, with the run masks repeated in
    // both halves, restores both blocks' invariant bits: run j moves bits
    // up by shift_j, and a half's bits never reach the other half's places
    // (the lowest upper-half place of run j is bit 16 + shift_j + its
    // source bit), so a raw half or the bits past a payload cannot leak.
    const uint32_t bv2 = (uint32_t)cd.bitval * 0x10001u;
    const uint32_t sh = 2u * (lane & 15u);
    const uint32_t sh1 = sh + 1u;
    const uint32_t hsel = 4u * (lane >> 4);
    // the lane's bit cursor, u plus 32 bits per lane below it, kept in a
    // vector register and advanced once per step
    uint32_t ul = u + 32u * lane;
    uint32_t* out_w = reinterpret_cast<uint32_t*>(out);
    auto pair = [&](uint32_t k0, bool ragged) {
      // the lane's header word, q + l/16, from the lane of hw holding it
      const uint32_t q = (k0 - lo) / 32;
      const uint32_t hs = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * q + hsel), (int)hw);
      // all ones / zero: the first / second block of the pair stripped
      const uint32_t m0 = (uint32_t)__builtin_amdgcn_sbfe((int)hs, sh, 1);
      const uint32_t m1 = (uint32_t)__builtin_amdgcn_sbfe((int)hs, sh1, 1);
      const bool s0 = m0 != 0u, s1 = m1 != 0u;
      const unsigned long long e = __ballot(s0), o = __ballot(s1);
      const bool valid = !ragged || k0 + 2u * lane < hi;
      const uint32_t below = bits_below_lane_acc((uint32_t)o, (uint32_t)(o >> 32),
                                                 bits_below_lane((uint32_t)e, (uint32_t)(e >> 32)));
      const uint32_t rel = valid ? (uint32_t)__mul24(negp, (int)below) + ul : 0u;
      // the window word index as an opaque value: its LDS address is then one
      // shift-add on it, not a shift, an and and an add on rel
      uint32_t wi = __builtin_amdgcn_ubfe(rel, 5, 27);
      asm volatile("" : "+v"(wi));
      const uint32_t v = __builtin_amdgcn_alignbit(lds[wi + 1], lds[wi], rel & 31u);
      // low half: the first payload; high half: the second one, which starts
      // 16 - p bits on when the first block is stripped, else 16
      const uint32_t y = select_bits(0xFFFFu, v, v << (cd.p & m0));
      uint32_t dep = bv2;
      if constexpr (NR >= 0) {
#pragma unroll
        for (int j = 0; j < NR; ++j) dep |= (y << cd.shift[j]) & ((uint32_t)cd.place[j] * 0x10001u);
      } else {
        for (uint32_t j = 0; j < cd.nruns; ++j)
          dep |= (y << cd.shift[j]) & ((uint32_t)cd.place[j] * 0x10001u);
      }
      const uint32_t sel = select_bits(0xFFFFu, m0, m1);
      if (valid) __builtin_nontemporal_store(select_bits(sel, dep, y), out_w + k0 / 2 + lane);
      // the step's advance is scalar work; kept opaque so that it is one
      // vector add, not a subtract and an add of a constant
      uint32_t adv = 16u * 2u * kWave - cd.p * (uint32_t)(__popcll(e) + __popcll(o));
      asm volatile("" : "+s"(adv));
      ul += adv;
    };
    if (hi - lo == kFull && seg == kFull) {
#pragma unroll
      for (uint32_t c = 0; c < kFull / (2 * kWave); ++c) pair(lo + c * 2 * kWave, false);
    } else {
      const uint32_t full_hi = lo + ((hi - lo) & ~(uint32_t)(2 * kWave - 1));
      uint32_t k0 = lo;
      for (; k0 < full_hi; k0 += 2 * kWave) pair(k0, false);
      if (k0 < hi) pair(k0, true);
    }
    wave_lds_sync();
    return;
  }
  const uint32_t wl = W * lane;
  // one 64-block chunk: lane l restores block k0 + l; `ragged` only for the
  // last chunk of a segment shorter than a whole number of chunks
  auto chunk = [&](uint32_t k0, bool ragged) {
    const uint32_t q = (k0 - lo) / 32;
    const uint32_t h_lo = __builtin_amdgcn_readlane(hw, q);
    const uint32_t h_hi = __builtin_amdgcn_readlane(hw, q + 1);
    const bool valid = !ragged || k0 + lane < hi;
    const uint32_t rel =
        valid ? (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + (u + wl) : 0u;
    const T v = lds_payload<T>(lds, rel);
    const bool stripped =
        __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
    const T x = stripped ? deposit_wide<T, NR>(v, cd) : v;
    if (valid) __builtin_nontemporal_store(x, out + k0 + lane);
    u += W * kWave - cd.p * (uint32_t)__popcll(((unsigned long long)h_hi << 32) | h_lo);
  };
  if (hi - lo == kFull && seg == kFull) {
#pragma unroll
    for (uint32_t c = 0; c < kFull / kWave; ++c) chunk(lo + c * kWave, false);
  } else {
    const uint32_t full_hi = lo + ((hi - lo) & ~(uint32_t)(kWave - 1));
    uint32_t k0 = lo;
    for (; k0 < full_hi; k0 += kWave) chunk(k0, false);
    if (k0 < hi) chunk(k0, true);
  }
  wave_lds_sync();
}

// [IBP] Decompression for W = 16 / 64: one wave per (row, segment of `seg`
// blocks), in the three row-source modes of the 32-bit kernels.
template <typename T, int MODE, int NR>
__global__ __launch_bounds__(kBlockThreads) void decode_wide_kernel(
    WideCodec<T> cd, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    const uint32_t* __restrict__ arena, const unsigned long long* __restrict__ cache_loc,
    uint64_t n_rows, uint64_t n_tasks, uint32_t nseg, uint32_t seg, T* __restrict__ dst,
    int vec, int remap) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerBlock][kSegLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint32_t g = gridDim.x;
  for (uint64_t wg = remap ? xcd_remap(blockIdx.x, g) : blockIdx.x; ; wg += g) {
    const uint64_t task = wg * kWavesPerBlock + wave;
    if (task >= n_tasks) break;
    const uint64_t i = task / nseg;
    const uint32_t s = (uint32_t)(task - i * nseg);
    decode_wide_task<T, MODE, NR>(cd, cd.n, cd.nw, slots, flags, ids, arena, cache_loc, n_rows,
                                  i, s, seg, dst, vec, lds, lane);
  }
}

// [IBP] Decompression for W = 16 / 64 of several tensors that share one
// Mask/Bitval in one launch, as decode_batch_kernel for W = 32: the segment
// tasks of every tensor one after the other, each mapped to its tensor by the
// running task counts.
template <typename T, int NR>
__global__ __launch_bounds__(kBlockThreads) void decode_wide_batch_kernel(WideCodec<T> cd,
                                                                          Batch batch,
                                                                          uint32_t seg) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerBlock][kSegLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint64_t n_tasks = batch.end[batch.count - 1];
  const uint32_t g = gridDim.x;
  for (uint64_t wg = blockIdx.x; ; wg += g) {
    const uint64_t task = wg * kWavesPerBlock + wave;
    if (task >= n_tasks) break;
    uint32_t t = 0;
    while (task >= batch.end[t]) ++t;
    const BatchTensor& bt = batch.t[t];
    const uint64_t local = task - (t ? batch.end[t - 1] : 0ull);
    const uint64_t i = local / bt.nseg;
    const uint32_t s = (uint32_t)(local - i * bt.nseg);
    decode_wide_task<T, kModeTable, NR>(cd, bt.n, bt.nw, bt.slots, bt.flags, nullptr, nullptr,
                                        nullptr, 0, i, s, seg, reinterpret_cast<T*>(bt.dst),
                                        (int)bt.vec, lds, lane);
  }
}

// [IBP] Decompression with 64-bit blocks of rows of 512 bytes to 2 KiB (32 * NCH
// blocks, NCH = 2, 4, 8), 16-byte aligned: the row pipeline of the 32-bit
// decoder with 64-bit stores (SLOT: the whole-slot pipeline, for p <= 16).  A compressed row's stream is nb + 64 nb - p m
// bits (nb blocks, m stripped); per 64-block chunk a lane's payload starts at
// u + 64 lane - p * (stripped blocks of the chunk below the lane) and is read
// from three LDS words with two funnel shifts.
template <int MODE, int NR, int NCH, bool SLOT = false>
__global__ __launch_bounds__(kBlockThreads) void decode_pipe64_kernel(
    WideCodec<uint64_t> cd, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    uint64_t n_rows, uint32_t n_out, uint32_t* __restrict__ dst) {
  using P = RowPipe<NCH>;
  constexpr uint32_t n = P::n;   // words of a row
  constexpr uint32_t nb = n / 2;  // 64-bit blocks of a row
  __shared__ __attribute__((aligned(16)))
  uint32_t lds_all[kWavesPerBlock][SLOT ? (NCH >= 4 ? n : 256u) + 4u : P::kLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const uint32_t stride = gridDim.x * kWavesPerBlock;
  const uint32_t i = blockIdx.x * kWavesPerBlock + wave;
  if (i >= n_out) return;
  const int negp = -(int)cd.p;
  const uint32_t l64 = 64u * lane;
  auto stream_words = [&](uint32_t win) -> uint32_t {
    const uint32_t m = wave_sum(__popc(lane < nb / 32 ? win : 0u));
    return (nb + 64u * nb - cd.p * m + 31u) >> 5;
  };
  auto decode = [&](uint32_t win, unsigned long long* x) {
    uint32_t u = nb;
#pragma unroll
    for (int c = 0; c < NCH / 2; ++c) {
      const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
      const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
      const uint32_t rel = (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + (u + l64);
      const uint64_t v = lds_payload<uint64_t>(lds, rel);
      const bool stripped =
          __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
      x[c] = stripped ? deposit_wide<uint64_t, NR>(v, cd) : v;
      u += 64u * kWave - cd.p * (uint32_t)__popcll(((unsigned long long)h_hi << 32) | h_lo);
    }
  };
  row_pipeline<NCH, MODE == kModeGather, SLOT, 2>(slots, flags, ids, n_rows, n_out, dst, lds, i,
                                                  stride, stream_words, decode);
}

// ---------------------------------------------------- per-position metadata --
//
// One Mask/Bitval per block position of a row (W = 32).  Lengths now differ
// per position, so the offset of a lane's payload is a real prefix sum: the
// DPP wave scan of (stripped ? p_k : 0) over the chunk.  The kept bits come
// out and go back with five shift-and-select steps whose masks depend only
// on ~Mask_k (parallel suffix method, Hacker's Delight sections 7-4 and 7-5)
// and are precomputed in the position table.  A row's stripped bits are
// summed from the header words and six bit planes of p per chunk on the
// scalar unit, so its stream length is known before the stream is fetched.

struct PosEntry {
  uint32_t mask, bitval, p;
  uint32_t sfx[5];
};
static_assert(sizeof(PosEntry) == 32, "position table entries are 32 bytes");
constexpr uint32_t kPlaneWords = 8;  // u64 per chunk: 6 planes of p, 2 zero

__device__ __forceinline__ PosEntry load_entry(const PosEntry* t, uint32_t k) {
  const uint4* q = reinterpret_cast<const uint4*>(t + k);
  const uint4 a = q[0], b = q[1];
  return PosEntry{a.x, a.y, a.z, {a.w, b.x, b.y, b.z, b.w}};
}

// Kept bits of x (under ~mask) packed to the bottom, and the inverse.
__device__ __forceinline__ uint32_t extract_pos(uint32_t x, const PosEntry& e) {
  x &= ~e.mask;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t t = x & e.sfx[i];
    x = (x ^ t) | (t >> (1u << i));
  }
  return x;
}

__device__ __forceinline__ uint32_t deposit_pos(uint32_t v, const PosEntry& e) {
#pragma unroll
  for (int i = 4; i >= 0; --i) v = select_bits(e.sfx[i], v << (1u << i), v);
  return select_bits(e.mask, e.bitval, v);
}

// Inclusive prefix sum over the 64 lanes (DPP row shifts, then row
// broadcasts across the four rows of 16 lanes).
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Sum of p over the stripped blocks of one chunk, from its 64-bit header and
// the chunk's planes of p (scalar).
__device__ __forceinline__ uint32_t chunk_stripped_bits(unsigned long long h,
                                                        const unsigned long long* planes) {
  uint32_t s = 0;
#pragma unroll
  for (int t = 0; t < 6; ++t) s += (uint32_t)__popcll(h & planes[t]) << t;
  return s;
}

// Per-position ones counts: one wave per (64 positions, range of rows);
// lane = position, rows summed bit-sliced 32 at a time, then added to
// counts[k * 32 + b] with one atomic per set count.
__global__ __launch_bounds__(kBlockThreads) void count_positions_kernel(
    const uint32_t* __restrict__ sample, uint64_t n_srows, uint32_t n, uint32_t n_chunks,
    uint32_t rows_per_task, uint64_t n_tasks, uint32_t* __restrict__ counts) {
  const uint32_t lane = lane_id();
  const uint64_t task = (uint64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave);
  if (task >= n_tasks) return;
  const uint32_t c = (uint32_t)(task % n_chunks);
  const uint64_t r0 = (task / n_chunks) * rows_per_task;
  const uint64_t r1 = std::min<uint64_t>(n_srows, r0 + rows_per_task);
  const uint32_t k = c * kWave + lane;
  const bool valid = k < n;
  uint32_t acc[12];  // rows_per_task < 2^12
#pragma unroll
  for (int j = 0; j < 12; ++j) acc[j] = 0;
  for (uint64_t r = r0; r < r1; r += kCountWords) {
    uint32_t w[kCountWords];
#pragma unroll
    for (int j = 0; j < kCountWords; ++j)
      w[j] = (valid && r + j < r1) ? sample[(r + j) * n + k] : 0u;
    uint32_t s[6];
    sliced_count32(w, s);
    sliced_accumulate<12, 6>(acc, s);
  }
  if (!valid) return;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 12; ++j) cnt += __builtin_amdgcn_ubfe(acc[j], b, 1) << j;
    if (cnt) atomicAdd(&counts[(uint64_t)k * 32 + b], cnt);
  }
}

// [IBP] Compression with per-position metadata, one workgroup per row (the
// stream is assembled in LDS as in compress_kernel).
template <uint32_t MAXW>
__global__ __launch_bounds__(kBlockThreads) void compress_positional_kernel(
    const PosEntry* __restrict__ table, uint32_t n, uint64_t n_rows, const uint32_t* src,
    uint32_t* slots, unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits) {
  __shared__ uint32_t buf[MAXW + 4];
  __shared__ uint32_t chunk_pre[MAXW / kWave + 1];
  __shared__ uint32_t total_s;
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  const uint32_t nchunks = (n + kWave - 1) / kWave;
  for (uint64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    const uint32_t* x_row = src + row * n;
    uint32_t* s_row = slots + row * n;
    for (uint32_t j = threadIdx.x; j < n + 4; j += kBlockThreads) buf[j] = 0;
    __syncthreads();
    for (uint32_t c = wave; c < nchunks; c += kWavesPerBlock) {  // header, chunk sums
      const uint32_t k = c * kWave + lane;
      const bool valid = k < n;
      uint32_t x = 0, mask = 0, bitval = 0, p = 0;
      if (valid) {
        x = x_row[k];
        mask = table[k].mask;
        bitval = table[k].bitval;
        p = table[k].p;
      }
      const bool match = valid && (x & mask) == bitval;
      const unsigned long long h = __ballot(match);
      const uint32_t s = wave_sum(match ? p : 0u);
      if (lane == 0) {
        chunk_pre[c] = s;
        buf[2 * c] = (uint32_t)h;
        buf[2 * c + 1] = (uint32_t)(h >> 32);
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t carry = 0;
      for (uint32_t b0 = 0; b0 < nchunks; b0 += kWave) {
        const uint32_t c = b0 + lane;
        const uint32_t v = c < nchunks ? chunk_pre[c] : 0u;
        const uint32_t inc = wave_inclusive_scan(v, lane);
        if (c < nchunks) chunk_pre[c] = carry + inc - v;
        carry += __shfl(inc, kWave - 1, kWave);
      }
      if (lane == 0) total_s = carry;
    }
    __syncthreads();
    const uint32_t c_bits = n + 32u * n - total_s;
    const bool flag = c_bits < 32u * n;
    if (!flag) {
      for (uint32_t j = threadIdx.x; j < n; j += kBlockThreads) s_row[j] = x_row[j];
    } else {
      for (uint32_t c = wave; c < nchunks; c += kWavesPerBlock) {
        const uint32_t k = c * kWave + lane;
        const bool valid = k < n;
        const PosEntry e = load_entry(table, valid ? k : 0u);
        const uint32_t x = valid ? x_row[k] : 0u;
        const bool match = valid && (x & e.mask) == e.bitval;
        const uint32_t v = match ? e.p : 0u;
        const uint32_t incl = wave_scan_incl(v);
        if (valid) {
          const uint32_t off = n + 32u * k - (chunk_pre[c] + incl - v);
          const uint32_t len = 32u - v;
          const uint32_t pay = match ? extract_pos(x, e) : x;
          if (len) {
            const uint32_t sh = off & 31u, wi = off >> 5;
            atomicOr(&buf[wi], pay << sh);
            if (sh + len > 32u) atomicOr(&buf[wi + 1], pay >> (32u - sh));
          }
        }
      }
      __syncthreads();
      const uint32_t words = (c_bits + 31u) >> 5;
      for (uint32_t j = threadIdx.x; j < words; j += kBlockThreads) __builtin_nontemporal_store(buf[j], &s_row[j]);
    }
    if (threadIdx.x == 0) {
      put_flag_bits(flags, row, 1u, flag ? 1ull : 0ull, n_rows);
      if (row_bits) row_bits[row] = c_bits;
    }
    // the LDS stream is reused only by a next row; after the last one the
    // workgroup ends without waiting for its stores (a barrier would)
    if (row + gridDim.x < n_rows) __syncthreads();
  }
}

// [IBP] Decompression with per-position metadata: one wave per output row,
// its segments of kSegBlocks blocks in order (a running count of stripped
// bits carries the stream offset from one segment to the next).  With
// TAB > 0 (rows of at most TAB blocks) the workgroup first copies the
// position entries into LDS field by field (conflict-free reads of one field
// of 64 consecutive positions), so that the per-chunk entry reads are LDS
// reads; the grid is then kept small and each wave decodes many rows.
template <bool GATHER, uint32_t TAB>
__global__ __launch_bounds__(kBlockThreads) void decode_positional_kernel(
    const PosEntry* __restrict__ table, uint32_t n, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    uint64_t n_rows, uint64_t n_out, uint32_t* __restrict__ dst, int vec) {
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerBlock][kSegLdsWords];
  __shared__ uint32_t tf[TAB > 0 ? 8 : 1][TAB > 0 ? TAB : 1];  // fields by position
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  const unsigned long long* planes =
      reinterpret_cast<const unsigned long long*>(table + n);  // after the n entries
  if constexpr (TAB > 0) {
    const uint32_t* g = reinterpret_cast<const uint32_t*>(table);
    for (uint32_t j = threadIdx.x; j < 8 * n; j += kBlockThreads) tf[j % 8][j / 8] = g[j];
    __syncthreads();
  }
  auto entry = [&](uint32_t k) -> PosEntry {
    if constexpr (TAB > 0)
      return PosEntry{tf[0][k], tf[1][k], tf[2][k], {tf[3][k], tf[4][k], tf[5][k], tf[6][k], tf[7][k]}};
    else
      return load_entry(table, k);
  };
  const uint64_t stride = (uint64_t)gridDim.x * kWavesPerBlock;
  for (uint64_t i = (uint64_t)blockIdx.x * kWavesPerBlock + wave;
       i < n_out; i += stride) {
    const uint64_t id = GATHER ? (uint64_t)ids[i] : i;
    uint32_t* out = dst + i * n;
    if (GATHER && id >= n_rows) {
      for (uint32_t j = lane; j < n; j += kWave) out[j] = 0u;
      continue;
    }
    const uint32_t* src = slots + id * n;
    if (!((flags[id >> 6] >> (id & 63)) & 1ull)) {
      if (vec) {
        const uint4* a = reinterpret_cast<const uint4*>(src);
        uint4* o = reinterpret_cast<uint4*>(out);
        for (uint32_t j = lane; j < n / 4; j += kWave) o[j] = a[j];
      } else {
        for (uint32_t j = lane; j < n; j += kWave) out[j] = src[j];
      }
      continue;
    }
    uint32_t carry = 0;  // sum of p over the stripped blocks before the segment
    for (uint32_t lo = 0; lo < n; lo += kSegBlocks) {
      const uint32_t hi = min(n, lo + kSegBlocks);
      const uint32_t hw_n = (hi - lo + 31) / 32;
      uint32_t hw = 0;
      if (lane < hw_n) {
        const uint32_t t = lo / 32 + lane;
        hw = src[t];
        const uint32_t valid_bits = min(32u, hi - 32u * t);
        if (valid_bits < 32u) hw &= (1u << valid_bits) - 1u;
      }
      uint32_t s_seg = 0;
      for (uint32_t k0 = lo; k0 < hi; k0 += kWave) {
        const uint32_t q = (k0 - lo) / 32;
        // readlane yields an int: narrow to 32 bits before widening, or bit 31
        // of the low word would be sign-extended into the high word
        const uint32_t h_lo = __builtin_amdgcn_readlane(hw, q);
        const uint32_t h_hi = __builtin_amdgcn_readlane(hw, q + 1);
        const unsigned long long h = ((unsigned long long)h_hi << 32) | h_lo;
        s_seg += chunk_stripped_bits(h, planes + (uint64_t)(k0 / kWave) * kPlaneWords);
      }
      const uint32_t a = n + 32u * lo - carry;
      const uint32_t b = n + 32u * hi - (carry + s_seg);
      const uint32_t wb = min((b + 31u) >> 5, n);
      const uint32_t wa = min(a >> 5, wb);
      uint32_t base = wa;
      if (vec) {
        base = wa & ~3u;
        stage_window<5, true>(reinterpret_cast<const u32x4*>(src + base),
                              reinterpret_cast<u32x4*>(lds), (wb - base + 3u) / 4u, lane);
      } else {
        stage_window<4, true>(src + wa, lds, wb - wa, lane);
      }
      wave_lds_sync();
      uint32_t u = a - 32u * base;
      for (uint32_t k0 = lo; k0 < hi; k0 += kWave) {
        const uint32_t q = (k0 - lo) / 32;
        const uint32_t h_lo = __builtin_amdgcn_readlane(hw, q);
        const uint32_t h_hi = __builtin_amdgcn_readlane(hw, q + 1);
        const bool valid = k0 + lane < hi;
        const PosEntry e = entry(valid ? k0 + lane : 0u);
        const bool stripped =
            __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
        const uint32_t v = stripped ? e.p : 0u;
        const uint32_t incl = wave_scan_incl(v);
        const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
        const uint32_t rel = valid ? u + 32u * lane - (incl - v) : 0u;
        const uint32_t w = lds_bits(lds, rel);
        const uint32_t x = stripped ? deposit_pos(w, e) : w;
        if (valid) __builtin_nontemporal_store(x, out + k0 + lane);
        u += 32u * kWave - total;
      }
      carry += s_seg;
      wave_lds_sync();
    }
  }
}

// The first two runs of kept bits (~mask) of a uniform mask, as make_codec
// cuts them on the host: run j moves payload bits down by sh[j] into the
// positions place[j].  Returns the number of runs, 3 meaning three or more
// (then sh/place hold only the first two).  Scalar work, once per workgroup.
__device__ __forceinline__ uint32_t kept_runs2(uint32_t mask, uint32_t (&sh)[2],
                                               uint32_t (&place)[2]) {
  sh[0] = sh[1] = place[0] = place[1] = 0u;
  uint32_t keep = ~mask, at = 0, nr = 0;
  while (keep != 0u && nr < 3u) {
    const uint32_t b = (uint32_t)__builtin_ctz(keep);
    const uint32_t rest = ~(keep >> b);
    const uint32_t len = rest == 0u ? 32u - b : (uint32_t)__builtin_ctz(rest);
    const uint32_t pl = (len >= 32u ? ~0u : ((1u << len) - 1u)) << b;
    if (nr < 2u) {
      sh[nr] = b - at;
      place[nr] = pl;
    }
    at += len;
    keep &= ~pl;
    ++nr;
  }
  return nr;
}

// The position entries of rows of n blocks staged into LDS field by field
// (tf[0] Mask, tf[1] Bitval, tf[2..6] the five parallel-suffix masks), so
// that a wave reads one field of 64 consecutive positions without bank
// conflicts; a 32-byte entry per lane would put lanes 4 apart on one bank.
// Every thread of the workgroup takes part (ends with a barrier).
template <uint32_t n>
__device__ __forceinline__ void stage_pos_table(const PosEntry* __restrict__ table,
                                                uint32_t (*tf)[n]) {
  const u32x4* g = reinterpret_cast<const u32x4*>(table);
  for (uint32_t k = threadIdx.x; k < n; k += blockDim.x) {
    const u32x4 a = g[2 * k], b = g[2 * k + 1];  // {mask, bitval, p, sfx0}, {sfx1..4}
    tf[0][k] = a.x;
    tf[1][k] = a.y;
    tf[2][k] = a.w;
    tf[3][k] = b.x;
    tf[4][k] = b.y;
    tf[5][k] = b.z;
    tf[6][k] = b.w;
  }
  __syncthreads();
}

template <uint32_t n>
__device__ __forceinline__ PosEntry pos_entry(const uint32_t (*tf)[n], uint32_t k) {
  return PosEntry{tf[0][k], tf[1][k], 0u, {tf[2][k], tf[3][k], tf[4][k], tf[5][k], tf[6][k]}};
}

// p of the lane's position in each chunk c, as byte c % 4 of pp[c / 4].
template <int NCH>
__device__ __forceinline__ void pack_pos_p(const uint32_t (*tf)[NCH * kWave], uint32_t lane,
                                           uint32_t* pp) {
#pragma unroll
  for (int w = 0; w < (NCH + 3) / 4; ++w) pp[w] = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    pp[c / 4] |= (uint32_t)__popc(tf[0][c * kWave + lane]) << (8 * (c % 4));
}

// [IBP] Compression with per-position metadata of rows of exactly 64 * NCH
// blocks, one wave per row (the scheme of compress_rows_kernel): the row is
// read once into registers, each chunk's match ballot is its header word,
// the bit offset of a block's payload is n + 32 k minus the stripped p of
// the blocks before it (a scalar carry across chunks plus a DPP wave scan
// within one), and the payloads are ORed into a wave-private LDS stream that
// is then written with coalesced stores.  In place is safe: every load of a
// row completes before its first store.
template <int NCH, int WPB>
__global__ __launch_bounds__(WPB * kWave) void compress_pos_rows_kernel(
    const PosEntry* __restrict__ table, uint64_t n_rows, const uint32_t* src, uint32_t* slots,
    unsigned long long* __restrict__ flags, uint32_t* __restrict__ row_bits, uint32_t pad) {
  constexpr uint32_t n = NCH * kWave;
  __shared__ uint32_t tf[7][n];
  __shared__ uint32_t lds_all[WPB][n + 4];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* buf = lds_all[wave];
  stage_pos_table<n>(table, tf);
  uint32_t pp[(NCH + 3) / 4];
  pack_pos_p<NCH>(tf, lane, pp);
  auto p_of = [&](int c) { return __builtin_amdgcn_ubfe(pp[c / 4], 8 * (c % 4), 8); };

  // Every position with one (Mask, Bitval): the image is the global one, and
  // the rows are compressed with the global arithmetic (offsets from the
  // stripped count by v_mbcnt, no scan; the extract masks in scalar
  // registers).  As in the decoder, only the kernels for rows of up to 512
  // blocks carry this path.
  if constexpr (NCH <= 8) {
    const uint32_t m0 = uniform(tf[0][0]), b0 = uniform(tf[1][0]);
    bool same = true;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      same = same && tf[0][c * kWave + lane] == m0 && tf[1][c * kWave + lane] == b0;
    if (__ballot(!same) == 0ull) {
      const uint32_t p = (uint32_t)__popc(m0);
      PosEntry e = pos_entry<n>(tf, 0);
      e.mask = m0;
      e.bitval = b0;
#pragma unroll
      for (int j = 0; j < 5; ++j) e.sfx[j] = uniform(e.sfx[j]);
      // with at most two runs of kept bits, the extract is a shift and an
      // and-or per run (as compress_rows_kernel's), else the five steps of
      // the position entries
      uint32_t rsh[2], rpl[2];
      const uint32_t nruns = kept_runs2(m0, rsh, rpl);
      const uint32_t sh0 = uniform(rsh[0]), sh1 = uniform(rsh[1]);
      const uint32_t kp0 = uniform(rpl[0] >> rsh[0]), kp1 = uniform(rpl[1] >> rsh[1]);
      auto encode = [&](auto extract) {
      compress_row_range(n_rows, wave, WPB, 32u * n, flags, row_bits, [&](uint64_t row) {
        const uint32_t* x_row = src + row * n;
        uint32_t* s_row = slots + row * n;
        uint32_t x[NCH];
        unsigned long long h[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) x[c] = __builtin_nontemporal_load(&x_row[c * kWave + lane]);
        uint32_t m = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          h[c] = __ballot((x[c] & m0) == b0);
          m += (uint32_t)__popcll(h[c]);
        }
        const uint32_t c_bits = n + 32u * n - p * m;
        const bool flag = c_bits < 32u * n;
        if (!flag) {
#pragma unroll
          for (int c = 0; c < NCH; ++c) s_row[c * kWave + lane] = x[c];
        } else {
          const uint32_t nw = store_words(s_row, (c_bits + 31u) >> 5, n, pad);
          for (uint32_t j = n / 32 + lane; j < nw + 1; j += kWave) buf[j] = 0u;
          if (lane < 2 * NCH) {
            uint32_t w = 0;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
              if (lane == 2u * c) w = (uint32_t)h[c];
              if (lane == 2u * c + 1) w = (uint32_t)(h[c] >> 32);
            }
            buf[lane] = w;
          }
          wave_lds_sync();
          uint32_t carry = 0;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const uint32_t lo = (uint32_t)h[c], hi = (uint32_t)(h[c] >> 32);
            const bool match = __builtin_amdgcn_inverse_ballot_w64(h[c]);
            const uint32_t off =
                n + 32u * (c * kWave + lane) - __umul24(p, carry + bits_below_lane(lo, hi));
            const uint32_t len = match ? 32u - p : 32u;
            const uint32_t pay = match ? extract(x[c]) : x[c];
            if (len) {
              const uint32_t sh = off & 31u, wi = off >> 5;
              atomicOr(&buf[wi], pay << sh);
              if (sh + len > 32u) atomicOr(&buf[wi + 1], pay >> (32u - sh));
            }
            carry += (uint32_t)__popcll(h[c]);
          }
          wave_lds_sync();
          for (uint32_t j = lane; j < nw; j += kWave) __builtin_nontemporal_store(buf[j], &s_row[j]);
          wave_lds_sync();
        }
        return c_bits;
      });
      };
      if (nruns <= 2u)
        encode([&](uint32_t v) { return ((v >> sh0) & kp0) | ((v >> sh1) & kp1); });
      else
        encode([&](uint32_t v) { return extract_pos(v, e); });
      return;
    }
  }

  compress_row_range(n_rows, wave, WPB, 32u * n, flags, row_bits, [&](uint64_t row) {
    const uint32_t* x_row = src + row * n;
    uint32_t* s_row = slots + row * n;
    uint32_t x[NCH];
    unsigned long long h[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) x[c] = __builtin_nontemporal_load(&x_row[c * kWave + lane]);
    uint32_t s_lane = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t k = c * kWave + lane;
      const bool match = (x[c] & tf[0][k]) == tf[1][k];
      h[c] = __ballot(match);
      s_lane += match ? p_of(c) : 0u;
    }
    const uint32_t c_bits = n + 32u * n - wave_sum(s_lane);
    const bool flag = c_bits < 32u * n;
    if (!flag) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) s_row[c * kWave + lane] = x[c];
    } else {
      const uint32_t nw = store_words(s_row, (c_bits + 31u) >> 5, n, pad);
      for (uint32_t j = n / 32 + lane; j < nw + 1; j += kWave) buf[j] = 0u;
      if (lane < 2 * NCH) {  // header word q = half (q & 1) of chunk q / 2's ballot
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          if (lane == 2u * c) w = (uint32_t)h[c];
          if (lane == 2u * c + 1) w = (uint32_t)(h[c] >> 32);
        }
        buf[lane] = w;
      }
      wave_lds_sync();
      uint32_t carry = 0;  // stripped p of the chunks before this one
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t k = c * kWave + lane;
        const bool match = __builtin_amdgcn_inverse_ballot_w64(h[c]);
        const uint32_t v = match ? p_of(c) : 0u;
        const uint32_t incl = wave_scan_incl(v);
        const uint32_t off = n + 32u * k - (carry + incl - v);
        const uint32_t len = 32u - v;
        const uint32_t pay = match ? extract_pos(x[c], pos_entry<n>(tf, k)) : x[c];
        if (len) {
          const uint32_t sh = off & 31u, wi = off >> 5;
          atomicOr(&buf[wi], pay << sh);
          if (sh + len > 32u) atomicOr(&buf[wi + 1], pay >> (32u - sh));
        }
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
      }
      wave_lds_sync();
      for (uint32_t j = lane; j < nw; j += kWave) __builtin_nontemporal_store(buf[j], &s_row[j]);
      wave_lds_sync();
    }
    return c_bits;
  });
}

// [IBP] Decompression with per-position metadata for rows of exactly
// 64 * NCH blocks (NCH = 2, 4, 8, 16), 16-byte aligned: the row pipeline of
// run_row_pipeline.  The position entries are copied once per workgroup of
// WPB waves into LDS, field by field (Mask, Bitval, the five deposit masks: a
// wave reads one field of 64 consecutive positions, conflict free; a 32-byte
// entry per lane would put lanes 4 apart on the same bank), and each lane's
// p values are packed as bytes in registers.  A row's stripped-bit total,
// which gives its stream length, is a per-lane sum over the chunks of p where
// the header bit is set (the header word used as a lane mask) and one wave
// sum; a payload's offset within a chunk is a DPP wave scan of the stripped
// p values.
template <bool GATHER, int NCH, int WPB>
__global__ __launch_bounds__(WPB * kWave) void decode_pos_pipe_kernel(
    const PosEntry* __restrict__ table, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    uint64_t n_rows, uint32_t n_out, uint32_t* __restrict__ dst) {
  using P = RowPipe<NCH>;
  constexpr uint32_t n = P::n;
  constexpr int PW = (NCH + 3) / 4;  // registers of packed p bytes
  __shared__ uint32_t tf[7][n];      // Mask, Bitval, sfx[0..4] by position
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[WPB][P::kLdsWords];
  const uint32_t lane = lane_id();
  const uint32_t wave = uniform(threadIdx.x / kWave);
  uint32_t* lds = lds_all[wave];
  stage_pos_table<n>(table, tf);
  uint32_t pp[PW];
  pack_pos_p<NCH>(tf, lane, pp);
  auto p_of = [&](int c) { return __builtin_amdgcn_ubfe(pp[c / 4], 8 * (c % 4), 8); };
  auto entry = [&](uint32_t k) { return pos_entry<n>(tf, k); };
  const uint32_t stride = gridDim.x * WPB;
  const uint32_t i = blockIdx.x * WPB + wave;
  if (i >= n_out) return;
  const uint32_t l32 = 32u * lane;

  // Every position with one (Mask, Bitval)?  Then the image is the one global
  // metadata gives, byte for byte, and the rows decode as such: offsets from
  // the stripped count (v_mbcnt) and one deposit with masks in scalar
  // registers, or for Mask = all ones the word-aligned copy of the global
  // decoder.  Tables whose positions differ take the general path below.
  // Rows of 1024 blocks keep the general path only: with these paths beside
  // it, its register allocation made it 4% slower (measured on KV pages).
  if constexpr (NCH <= 8) {
    const uint32_t m0 = uniform(tf[0][0]), b0 = uniform(tf[1][0]);
    bool same = true;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      same = same && tf[0][c * kWave + lane] == m0 && tf[1][c * kWave + lane] == b0;
    if (__ballot(!same) == 0ull) {
      const uint32_t p = (uint32_t)__popc(m0);
      const int negp = -(int)p;
      auto stream_words = [&](uint32_t win) -> uint32_t {
        const uint32_t m = wave_sum(__popc(lane < n / 32 ? win : 0u));
        return (n + 32u * n - p * m + 31u) >> 5;
      };
      if (p == 32) {
        // a stripped block is Bitval and every other payload is one whole
        // stream word: word index = header words + unstripped blocks before it
        auto decode = [&](uint32_t win, uint32_t* x) {
          uint32_t uw = n / 32;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
            const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
            const unsigned long long h = ((unsigned long long)h_hi << 32) | h_lo;
            const unsigned long long kept = ~h;
            const uint32_t v =
                lds[bits_below_lane_acc((uint32_t)kept, (uint32_t)(kept >> 32), uw)];
            x[c] = __builtin_amdgcn_inverse_ballot_w64(h) ? b0 : v;
            uw += (uint32_t)__popcll(kept);
          }
        };
        row_pipeline<NCH, GATHER, false>(slots, flags, ids, n_rows, n_out, dst, lds, i, stride,
                                         stream_words, decode);
      } else {
        // the kept bits ~m0 as runs, at most two taken (sign and mantissa
        // around an exponent field): then the deposit is a shift and an
        // and-or per run, as in the global decoder; more runs keep the five
        // shift-and-select steps of the position entries
        uint32_t rsh[2], rpl[2];
        const uint32_t nruns = kept_runs2(m0, rsh, rpl);
        if (nruns <= 2u) {
          const uint32_t sh0 = uniform(rsh[0]), sh1 = uniform(rsh[1]);
          const uint32_t pl0 = uniform(rpl[0]), pl1 = uniform(rpl[1]);
          auto decode = [&](uint32_t win, uint32_t* x) {
            uint32_t u = n;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
              const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
              const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
              const unsigned long long h = ((unsigned long long)h_hi << 32) | h_lo;
              const uint32_t rel =
                  (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + (u + l32);
              const uint32_t w = lds_bits(lds, rel);
              const uint32_t d = b0 | ((w << sh0) & pl0) | ((w << sh1) & pl1);
              x[c] = __builtin_amdgcn_inverse_ballot_w64(h) ? d : w;
              u += 32u * kWave - p * (uint32_t)__popcll(h);
            }
          };
          // few invariant bits: whole slots, as the global decoder fetches them
          if (p <= kSlotPipeMaxP)
            row_pipeline<NCH, GATHER, true>(slots, flags, ids, n_rows, n_out, dst, lds, i,
                                            stride, stream_words, decode);
          else
            row_pipeline<NCH, GATHER, false>(slots, flags, ids, n_rows, n_out, dst, lds, i,
                                             stride, stream_words, decode);
          return;
        }
        PosEntry e = pos_entry<n>(tf, 0);
        e.mask = m0;
        e.bitval = b0;
#pragma unroll
        for (int j = 0; j < 5; ++j) e.sfx[j] = uniform(e.sfx[j]);
        auto decode = [&](uint32_t win, uint32_t* x) {
          uint32_t u = n;
#pragma unroll
          for (int c = 0; c < NCH; ++c) {
            const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
            const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
            const unsigned long long h = ((unsigned long long)h_hi << 32) | h_lo;
            const uint32_t rel =
                (uint32_t)__mul24(negp, (int)bits_below_lane(h_lo, h_hi)) + (u + l32);
            const uint32_t w = lds_bits(lds, rel);
            x[c] = __builtin_amdgcn_inverse_ballot_w64(h) ? deposit_pos(w, e) : w;
            u += 32u * kWave - p * (uint32_t)__popcll(h);
          }
        };
        // few invariant bits: whole slots, as the global decoder fetches them
        if (p <= kSlotPipeMaxP)
          row_pipeline<NCH, GATHER, true>(slots, flags, ids, n_rows, n_out, dst, lds, i, stride,
                                          stream_words, decode);
        else
          row_pipeline<NCH, GATHER, false>(slots, flags, ids, n_rows, n_out, dst, lds, i, stride,
                                           stream_words, decode);
      }
      return;
    }
  }

  auto stream_words = [&](uint32_t win) -> uint32_t {
    uint32_t s_lane = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * c);
      const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * c + 1);
      const bool stripped =
          __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
      s_lane += stripped ? p_of(c) : 0u;
    }
    return (n + 32u * n - wave_sum(s_lane) + 31u) >> 5;
  };
  // Two chunks share one wave scan: chunk c's stripped p in the low half of
  // a word, chunk c + 1's in the high half (a chunk's sum is at most 64 * 32,
  // so neither half carries into the other).  The pair's position entries
  // are read before the scan (the barrier keeps them there) and both stream
  // words before either deposit, so the LDS reads overlap; the deposit is
  // computed for every lane and then selected.
  auto decode = [&](uint32_t win, uint32_t* x) {
    uint32_t u = n;
#pragma unroll
    for (int c = 0; c < NCH; c += 2) {
      const PosEntry e[2] = {entry(c * kWave + lane), entry((c + 1) * kWave + lane)};
      __builtin_amdgcn_sched_barrier(0);
      bool st[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t h_lo = __builtin_amdgcn_readlane(win, 2 * (c + j));
        const uint32_t h_hi = __builtin_amdgcn_readlane(win, 2 * (c + j) + 1);
        st[j] = __builtin_amdgcn_inverse_ballot_w64(((unsigned long long)h_hi << 32) | h_lo);
      }
      const uint32_t v = (st[0] ? p_of(c) : 0u) | ((st[1] ? p_of(c + 1) : 0u) << 16);
      const uint32_t incl = wave_scan_incl(v);
      const uint32_t excl = incl - v;  // per half: no borrow, incl >= v in each
      const uint32_t tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      uint32_t w[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        w[j] = lds_bits(lds, (u + l32) - ((excl >> (16 * j)) & 0xffffu));
        u += 32u * kWave - ((tot >> (16 * j)) & 0xffffu);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t d = deposit_pos(w[j], e[j]);
        x[c + j] = st[j] ? d : w[j];
      }
    }
  };
  row_pipeline<NCH, GATHER, false>(slots, flags, ids, n_rows, n_out, dst, lds, i, stride,
                                   stream_words, decode);
}

// ------------------------------------------------------ packed cache ----
//
// [IBP] System integration, cache compression: rows kept in a GPU software
// cache are stored compressed.  The arena holds each cached row's stored
// words back to back at 16-byte boundaries; a 64-bit locator per entry (and,
// after filling, per table row) gives offset, word count and flag.  Planning
// is sizes -> tile sums -> scan of the tile sums -> offsets.

constexpr uint32_t kScanTile = 4096;                          // entries per scan workgroup
constexpr uint32_t kScanPerThread = kScanTile / kBlockThreads;  // 16

// 16-byte units an entry takes in the arena (0 when the row is not packed).
__device__ __forceinline__ unsigned long long loc_units(unsigned long long loc) {
  if (!(loc & IBP_LOC_RESIDENT)) return 0;
  return (((loc >> IBP_LOC_WORDS_SHIFT) & IBP_LOC_WORDS_MASK) + 3) / 4;
}

// Inclusive scan over the workgroup's threads (buf: kBlockThreads slots).
__device__ unsigned long long block_inclusive_scan(unsigned long long v, unsigned long long* buf) {
  buf[threadIdx.x] = v;
  __syncthreads();
  for (uint32_t d = 1; d < kBlockThreads; d <<= 1) {
    const unsigned long long t = threadIdx.x >= d ? buf[threadIdx.x - d] : 0ull;
    __syncthreads();
    buf[threadIdx.x] += t;
    __syncthreads();
  }
  return buf[threadIdx.x];
}

// One wave per entry: loc[e] = resident | compressed | words of row ids[e]
// (its offset comes later); 0 for an id outside the table.  The words of a
// compressed row of n blocks follow from its header: ceil((n + W*n - p*m) / 32).
__global__ __launch_bounds__(kBlockThreads) void cache_sizes_kernel(
    uint32_t n, uint32_t nw, uint32_t w_bits, uint32_t p, const uint32_t* __restrict__ slots,
    const unsigned long long* __restrict__ flags, const int64_t* __restrict__ ids,
    uint64_t n_rows, uint64_t n_ids, unsigned long long* __restrict__ loc) {
  const uint32_t lane = lane_id();
  const uint64_t nwaves = (uint64_t)gridDim.x * kWavesPerBlock;
  const uint32_t hw_n = (n + 31) / 32;
  for (uint64_t e = (uint64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave);
       e < n_ids; e += nwaves) {
    const uint64_t id = (uint64_t)ids[e];
    unsigned long long out = 0;
    if (id < n_rows) {
      const bool flag = (flags[id >> 6] >> (id & 63)) & 1ull;
      uint32_t words = nw;
      if (flag) {
        const uint32_t* src = slots + id * nw;
        uint32_t acc = 0;
        for (uint32_t t = lane; t < hw_n; t += kWave) {
          uint32_t h = src[t];
          if (t == hw_n - 1 && (n & 31u)) h &= (1u << (n & 31u)) - 1u;
          acc += __popc(h);
        }
        const uint64_t m = wave_sum(acc);
        words = (uint32_t)std::min<uint64_t>(
            ((uint64_t)n * (1 + w_bits) - (uint64_t)p * m + 31) >> 5, nw);
      }
      out = IBP_LOC_RESIDENT | (flag ? IBP_LOC_COMPRESSED : 0ull) |
            ((unsigned long long)words << IBP_LOC_WORDS_SHIFT);
    }
    if (lane == 0) loc[e] = out;
  }
}

// sums[t] = 16-byte units of the entries of scan tile t.
__global__ __launch_bounds__(kBlockThreads) void cache_tile_sums_kernel(
    const unsigned long long* __restrict__ loc, uint64_t n_ids,
    unsigned long long* __restrict__ sums) {
  __shared__ unsigned long long buf[kBlockThreads];
  const uint64_t base = (uint64_t)blockIdx.x * kScanTile;
  unsigned long long t = 0;
  for (uint32_t j = threadIdx.x; j < kScanTile; j += kBlockThreads)
    if (base + j < n_ids) t += loc_units(loc[base + j]);
  const unsigned long long incl = block_inclusive_scan(t, buf);
  if (threadIdx.x == kBlockThreads - 1) sums[blockIdx.x] = incl;
}

// Exclusive scan of sums[0, nt) in place, total in sums[nt]; one workgroup.
__global__ __launch_bounds__(kBlockThreads) void cache_scan_sums_kernel(
    unsigned long long* __restrict__ sums, uint32_t nt) {
  __shared__ unsigned long long buf[kBlockThreads];
  unsigned long long carry = 0;
  for (uint32_t t0 = 0; t0 < nt; t0 += kBlockThreads) {
    const uint32_t j = t0 + threadIdx.x;
    const unsigned long long v = j < nt ? sums[j] : 0ull;
    const unsigned long long incl = block_inclusive_scan(v, buf);
    if (j < nt) sums[j] = carry + incl - v;
    carry += buf[kBlockThreads - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) sums[nt] = carry;
}

// Adds each entry's arena offset (16-byte units) to its locator.
__global__ __launch_bounds__(kBlockThreads) void cache_offsets_kernel(
    unsigned long long* __restrict__ loc, uint64_t n_ids,
    const unsigned long long* __restrict__ sums) {
  __shared__ unsigned long long buf[kBlockThreads];
  const uint64_t base = (uint64_t)blockIdx.x * kScanTile + (uint64_t)threadIdx.x * kScanPerThread;
  unsigned long long lv[kScanPerThread];
  unsigned long long t = 0;
#pragma unroll
  for (uint32_t k = 0; k < kScanPerThread; ++k) {
    lv[k] = base + k < n_ids ? loc[base + k] : 0ull;
    t += loc_units(lv[k]);
  }
  const unsigned long long incl = block_inclusive_scan(t, buf);
  unsigned long long off = sums[blockIdx.x] + incl - t;
#pragma unroll
  for (uint32_t k = 0; k < kScanPerThread; ++k) {
    if (lv[k] & IBP_LOC_RESIDENT) {
      loc[base + k] = lv[k] | (off & IBP_LOC_OFFSET_MASK);
      off += loc_units(lv[k]);
    }
  }
}

// One wave per entry: copy the row's stored words into its arena entry (zero
// padded to 16 bytes) and point the row's table locator at it.  Entries
// that would end past the arena, or whose id left the table, are skipped.
__global__ __launch_bounds__(kBlockThreads) void cache_fill_kernel(
    uint32_t n, const uint32_t* __restrict__ slots, const int64_t* __restrict__ ids,
    const unsigned long long* __restrict__ entry_loc, uint64_t n_ids, uint64_t n_rows,
    uint32_t* __restrict__ arena, uint64_t arena_units,
    unsigned long long* __restrict__ cache_loc) {
  const uint32_t lane = lane_id();
  const uint64_t nwaves = (uint64_t)gridDim.x * kWavesPerBlock;
  for (uint64_t e = (uint64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave);
       e < n_ids; e += nwaves) {
    const unsigned long long l = entry_loc[e];
    const uint64_t id = (uint64_t)ids[e];
    if (!(l & IBP_LOC_RESIDENT) || id >= n_rows) continue;
    const uint32_t words = (uint32_t)((l >> IBP_LOC_WORDS_SHIFT) & IBP_LOC_WORDS_MASK);
    const uint64_t off = l & IBP_LOC_OFFSET_MASK;
    if (words > n || off + loc_units(l) > arena_units) continue;
    const uint32_t* src = slots + id * n;
    uint32_t* out = arena + off * 4;
    const uint32_t padded = (words + 3u) & ~3u;
    for (uint32_t j = lane; j < padded; j += kWave) out[j] = j < words ? src[j] : 0u;
    if (lane == 0) cache_loc[id] = l;
  }
}

// ------------------------------------------------------------- host ----

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return IBP_ERR_HIP;
}

// A HIP error already pending on the calling thread (left by earlier work) is
// reported as IBP_ERR_HIP and left pending.  Every entry point checks this
// before its first HIP call, so the errors it reads back afterwards, and the
// one it clears in is_host_memory, are its own.
int pending_hip_error() {
  const hipError_t e = hipPeekAtLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

int popcount32(uint64_t x) {
  int c = 0;
  for (; x; x &= x - 1) ++c;
  return c;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool width_supported(uint32_t w) { return w == 16 || w == 32 || w == 64; }

int check_metadata(const ibp_metadata* md) {
  if (!md) return IBP_ERR_INVALID_ARGUMENT;
  if (!width_supported(md->width_bits)) return IBP_ERR_UNSUPPORTED;
  if ((md->width_bits < 64 && (md->mask >> md->width_bits) != 0) ||
      (md->bitval & ~md->mask) != 0 ||
      (int)md->invariant_bits != popcount32(md->mask) || md->t_ppm > 1000000u)
    return IBP_ERR_INVALID_ARGUMENT;
  return IBP_OK;
}

// Rows are whole 32-bit words, and whole blocks for 64-bit blocks.
int check_rows(uint64_t n_rows, uint64_t row_bytes, uint32_t w_bits = 32) {
  if (row_bytes == 0 || row_bytes % 4 != 0 || row_bytes % (w_bits / 8) != 0)
    return IBP_ERR_LAYOUT;
  if (row_bytes > kMaxRowBytes) return IBP_ERR_UNSUPPORTED;
  if (n_rows > UINT64_MAX / row_bytes) return IBP_ERR_INVALID_ARGUMENT;
  return IBP_OK;
}

Codec make_codec(const ibp_metadata* md, uint64_t row_bytes) {
  Codec cd{};
  cd.mask = (uint32_t)md->mask;
  cd.bitval = (uint32_t)md->bitval;
  cd.p = md->invariant_bits;
  cd.n = (uint32_t)(row_bytes / 4);
  const uint32_t keep = ~cd.mask;
  uint32_t at = 0, nr = 0;
  for (uint32_t b = 0; b < 32;) {
    if (!((keep >> b) & 1u)) { ++b; continue; }
    uint32_t e = b;
    while (e < 32 && ((keep >> e) & 1u)) ++e;
    const uint32_t len = e - b;
    cd.runs.shift[nr] = b - at;
    cd.runs.place[nr] = (len == 32 ? ~0u : ((1u << len) - 1u)) << b;
    ++nr;
    at += len;
    b = e;
  }
  cd.runs.n = nr;
  return cd;
}

template <typename T>
WideCodec<T> make_wide_codec(const ibp_metadata* md, uint64_t row_bytes) {
  constexpr uint32_t W = WideCodec<T>::W;
  WideCodec<T> cd{};
  cd.mask = (T)md->mask;
  cd.bitval = (T)md->bitval;
  cd.p = md->invariant_bits;
  cd.n = (uint32_t)(row_bytes * 8 / W);
  cd.nw = (uint32_t)(row_bytes / 4);
  const uint64_t keep = ~md->mask & (W == 64 ? ~0ull : ((1ull << W) - 1));
  uint32_t at = 0, nr = 0;
  for (uint32_t b = 0; b < W;) {
    if (!((keep >> b) & 1u)) { ++b; continue; }
    uint32_t e = b;
    while (e < W && ((keep >> e) & 1u)) ++e;
    const uint32_t len = e - b;
    cd.shift[nr] = b - at;
    cd.place[nr] = (T)((len == 64 ? ~0ull : ((1ull << len) - 1)) << b);
    ++nr;
    at += len;
    b = e;
  }
  cd.nruns = nr;
  return cd;
}

uint32_t grid_for(uint64_t work_groups) {
  return (uint32_t)(work_groups < kMaxGrid ? work_groups : kMaxGrid);
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // per device, read once (0: not yet)

// Workgroups for a launch on the current device: mult per CU (8 workgroups of
// 4 waves fill a CU).
uint32_t workgroups_per_device(uint32_t mult) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();  // the failed query's own error
    return mult * 256u;
  }
  if (dev < 0 || dev >= kMaxDevices) return mult * 256u;
  int cus = g_cu_count[dev].load(std::memory_order_relaxed);
  if (!cus) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
  }
  return mult * (uint32_t)cus;
}

// Grid of a row-pipeline launch over `rows` rows: as many workgroups of `wpb`
// waves as stay resident (`per_cu` per CU), but enough that no wave has more
// than 64 rows (one group of row bookkeeping), and no more than one row per
// wave.
uint32_t row_pipe_grid(uint32_t rows, uint32_t wpb, uint32_t per_cu) {
  const uint64_t one_per_wave = (rows + wpb - 1) / wpb;
  const uint64_t groups = (rows + 64ull * wpb - 1) / (64ull * wpb);
  return (uint32_t)std::min<uint64_t>(
      one_per_wave, std::max<uint64_t>(groups, workgroups_per_device(per_cu)));
}

template <int NR, uint32_t MAXW>
void launch_compress_t(const Codec& cd, uint64_t n_rows, const void* src, void* slots,
                       uint64_t* flags, uint32_t* row_bits, int vec, hipStream_t st) {
  hipLaunchKernelGGL((compress_kernel<NR, MAXW>), dim3(grid_for(n_rows)),
                     dim3(kBlockThreads), 0, st, cd, n_rows, (const uint32_t*)src,
                     (uint32_t*)slots, (unsigned long long*)flags, row_bits, vec);
}

// 32 workgroups per compute unit (four times what stays resident), so the
// dispatcher balances the ranges; every wave gets the same number of rows.
template <int NR, int NCH>
void launch_compress_rows_t(const Codec& cd, uint64_t n_rows, const void* src, void* slots,
                            uint64_t* flags, uint32_t* row_bits, hipStream_t st) {
  const uint64_t wgs = (n_rows + kWavesPerBlock - 1) / kWavesPerBlock;
  const uint32_t grid = (uint32_t)std::min<uint64_t>(wgs, workgroups_per_device(32));
  hipLaunchKernelGGL((compress_rows_kernel<NR, NCH>), dim3(grid), dim3(kBlockThreads), 0, st,
                     cd, n_rows, (const uint32_t*)src, (uint32_t*)slots,
                     (unsigned long long*)flags, row_bits);
}

// Rows per workgroup of compress_wg_kernel over n_rows rows with `cap`
// resident workgroups: enough that every workgroup is resident, at most 64;
// with `bytes`, a multiple of 8 (whole flag bytes, no atomics), else any
// (fewer rows per workgroup, two flag atomics each).
uint32_t cwg_rows_per_wg(uint64_t n_rows, uint64_t cap, bool bytes) {
  const uint64_t fill = (n_rows + cap - 1) / cap;
  return (uint32_t)std::min<uint64_t>(64, bytes ? 8 * ((fill + 7) / 8) : fill);
}

// Row lengths (in 32-bit words) that the weight-row kernels take
// (compress_wg_kernel, compress_pair_wg_kernel).
bool cwg_row(uint32_t n) { return n == 2048 || n == 4096 || n == 7168 || n == 8192; }

// Running workgroup counts of a batch at per_wg rows per workgroup; the
// total is the grid.
uint32_t set_wg_ends(CompressBatch& b, uint32_t per_wg) {
  uint32_t wgs = 0;
  for (uint32_t e = 0; e < b.count; ++e) {
    wgs += (uint32_t)((b.t[e].n_rows + per_wg - 1) / per_wg);
    b.wg_end[e] = wgs;
  }
  return wgs;
}

// Rows of one entry of a batched compression launch at most.  Longer
// tensors (2^29 rows of 8 KiB are 4 TiB) are cut into entries of this many
// rows, a multiple of 64, so that each entry's flag bits start a flag word; a
// launch then has at most 16 * 2^29 rows and, with up to 64 rows per
// workgroup once the rows outnumber the resident workgroups, fewer than 2^28
// workgroups.
constexpr uint64_t kCompressEntryRows = 1ull << 29;

// One launch of compress_wg_kernel over the entries of `b` (rows of cd.n
// blocks, b.count >= 1, total_rows rows), as many workgroups as stay resident
// (a CU holds 8 workgroups of 4 waves and 160 KiB of LDS, which holds their
// rows' streams).  Measured on 4096-row matrices: 8 rows per workgroup (flag
// bytes) for 8 KiB rows, and for 28 KiB rows fewer (atomics; 8 leave too few
// workgroups).
template <int NR>
void launch_compress_wg(const Codec& cd, CompressBatch& b, uint64_t total_rows, hipStream_t st) {
#define IBP_CWG(CPW, WPB, BYTES)                                                           \
  {                                                                                         \
    constexpr uint32_t lds = (CPW == 8 ? 2u : 1u) * (CPW * kWave * WPB + 4u + WPB) * 4u;    \
    constexpr uint32_t per_cu = std::min(32u / WPB, (160u * 1024u) / lds);                  \
    const uint32_t per_wg =                                                                 \
        cwg_rows_per_wg(total_rows, workgroups_per_device(per_cu), BYTES);                  \
    const uint32_t wgs = set_wg_ends(b, per_wg);                                            \
    hipLaunchKernelGGL((compress_wg_kernel<NR, CPW, WPB>), dim3(wgs), dim3(WPB * kWave), 0,  \
                       st, cd, b, per_wg);                                                  \
  }
  switch (cd.n) {
    case 2048: IBP_CWG(8, 4, true); return;
    case 4096: IBP_CWG(16, 4, true); return;
    case 7168: IBP_CWG(28, 4, false); return;
    default: IBP_CWG(32, 4, false); return;  // 8192
  }
#undef IBP_CWG
}

// Appends the rows of one tensor (rows of `words` 32-bit words) to a batch of
// weight-row kernel entries, calling flush(b, total_rows) to launch whenever
// the batch is full.
template <typename Flush>
void add_compress_entries(CompressBatch& b, uint64_t& total_rows, uint32_t words,
                          uint64_t n_rows, const void* src, void* slots, uint64_t* flags,
                          uint32_t* row_bits, uint32_t pad, Flush flush) {
  for (uint64_t off = 0; off < n_rows; off += kCompressEntryRows) {
    if (b.count == kCompressBatchMax) {
      flush(b, total_rows);
      b.count = 0;
      total_rows = 0;
    }
    CompressTensor& e = b.t[b.count++];
    e.src = (const uint32_t*)src + off * words;
    e.slots = (uint32_t*)slots + off * words;
    e.flags = (unsigned long long*)flags + off / 64;
    e.row_bits = row_bits ? row_bits + off : nullptr;
    e.n_rows = std::min(kCompressEntryRows, n_rows - off);
    e.pad = pad;
    total_rows += e.n_rows;
  }
}


template <int NR>
void launch_compress_nr(const Codec& cd, uint64_t n_rows, const void* src, void* slots,
                        uint64_t* flags, uint32_t* row_bits, int vec, hipStream_t st) {
  switch (cd.n) {  // rows of 64 * NCH blocks: one wave per row
    case 128: return launch_compress_rows_t<NR, 2>(cd, n_rows, src, slots, flags, row_bits, st);
    case 256: return launch_compress_rows_t<NR, 4>(cd, n_rows, src, slots, flags, row_bits, st);
    case 512: return launch_compress_rows_t<NR, 8>(cd, n_rows, src, slots, flags, row_bits, st);
    case 1024: return launch_compress_rows_t<NR, 16>(cd, n_rows, src, slots, flags, row_bits, st);
    default: break;
  }
  // rows of 256 * CPW blocks for the common long-row sizes (LLM weight rows
  // of 4096 or 14336 bf16 values): the register-resident workgroup kernel
  if (cwg_row(cd.n)) {
    CompressBatch b{};
    uint64_t total = 0;
    auto flush = [&](CompressBatch& fb, uint64_t rows) { launch_compress_wg<NR>(cd, fb, rows, st); };
    add_compress_entries(b, total, cd.n, n_rows, src, slots, flags, row_bits, cd.pad, flush);
    flush(b, total);
    return;
  }
  // LDS window tiers: the whole row stream (<= n words) lives in LDS
  if (cd.n <= 1024)
    launch_compress_t<NR, 1024>(cd, n_rows, src, slots, flags, row_bits, vec, st);
  else if (cd.n <= 4096)
    launch_compress_t<NR, 4096>(cd, n_rows, src, slots, flags, row_bits, vec, st);
  else if (cd.n <= 8192)
    launch_compress_t<NR, 8192>(cd, n_rows, src, slots, flags, row_bits, vec, st);
  else
    launch_compress_t<NR, IBP_MAX_COMPRESS_ROW_BYTES / 4>(cd, n_rows, src, slots, flags,
                                                          row_bits, vec, st);
}

// Pointers of a decode launch; arena and cache_loc only for kModeCached.
struct DecodeArgs {
  const void* slots;
  const uint64_t* flags;
  const int64_t* ids;
  const void* arena;
  const uint64_t* cache_loc;
  uint64_t n_rows;
  uint64_t n_out;
  void* dst;
  int vec;
  bool host_image;  // slots in pinned host memory (read across the host link)
};

// Is p host memory (pinned, mapped for the device)?  A decode from such an
// image is bound by the host link's latency and request count rather than by
// HBM, and prefers more, smaller tasks.
bool is_host_memory(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    // memory HIP does not know: treat it as device memory.  The entry point
    // checked that no error was pending before this query, so this clears
    // only the query's own error.
    (void)hipGetLastError();
    return false;
  }
  return at.type == hipMemoryTypeHost;
}

template <int MODE, int NR>
void launch_decode_t(const Codec& cd, const DecodeArgs& a, hipStream_t st) {
  const uint32_t* arena = (const uint32_t*)a.arena;
  const unsigned long long* cloc = (const unsigned long long*)a.cache_loc;
  // an image in host memory, rows of >= 1024 blocks with kept bits: tasks of
  // 256 blocks, so that more and smaller reads cross the host link at once
  // (measured: KV page gather 1004 -> 933 us, 28 KiB weight rows 1020 ->
  // 981 us; the link ceiling then bounds both at 0.96-0.97)
  const bool small_tasks = a.host_image && NR != 0 && MODE != kModeCached && cd.n >= 1024;
  if (cd.n <= kSegBlocks && !small_tasks) {
    const uint64_t piece = 1ull << 30;
    for (uint64_t off = 0; off < a.n_out; off += piece) {
      const uint32_t cnt = (uint32_t)std::min<uint64_t>(piece, a.n_out - off);
      const uint64_t wgs = (cnt + kWavesPerBlock - 1) / kWavesPerBlock;
      // Grid size (measured on MI355X): with Mask = all ones (p = 32) the
      // streams of sparse rows fit the prefetched window and one row per wave
      // with many workgroups in flight is fastest, except through the cache,
      // whose locator adds a dependent load that two rows per wave overlap
      // (all-hit sparse gather: 22.2 against 23.2 us); rows of 1024 blocks do
      // best with 16 workgroups per CU; shorter dense rows, which need a
      // second load per row, profit most from the pipeline of a resident grid.
      const uint32_t mult =
          cd.p == 32 ? (MODE == kModeCached ? 32u : 64u) : (cd.n >= 1024 ? 16u : 8u);
      const uint32_t grid = (uint32_t)std::min<uint64_t>(wgs, workgroups_per_device(mult));
      // a full decompress is the identity gather: row `off + r` of the table
      const uint32_t* sl = (const uint32_t*)a.slots;
      const unsigned long long* fl = (const unsigned long long*)a.flags;
      if (MODE == kModeTable) {  // shift the table window; flags stay word aligned (piece % 64 == 0)
        sl += off * cd.n;
        fl += off / 64;
      }
      const int64_t* id_p = MODE != kModeTable ? a.ids + off : a.ids;
      uint32_t* out_p = (uint32_t*)a.dst + off * cd.n;
#define IBP_ROWS(NCH)                                                                     \
  hipLaunchKernelGGL((decode_rows_kernel<MODE, NR, NCH>), dim3(grid), dim3(kBlockThreads), \
                     0, st, cd, sl, fl, id_p, arena, cloc, a.n_rows, cnt, out_p, a.vec)
#define IBP_PIPE(NCH)                                                                      \
  if (slot_pipe)                                                                            \
    hipLaunchKernelGGL((decode_pipe_kernel<MODE, NR, NCH, true>),                           \
                       dim3(pipe_grid), dim3(kBlockThreads), 0, st, cd, sl, fl, id_p, a.n_rows, \
                       cnt, out_p);                                                           \
  else                                                                                      \
    hipLaunchKernelGGL((decode_pipe_kernel<MODE, NR, NCH>),                                 \
                       dim3(pipe_grid), dim3(kBlockThreads), 0, st, cd, sl, fl, id_p, a.n_rows, \
                       cnt, out_p)
      // rows of 128-512 blocks with some invariant bits kept, 16-byte
      // aligned, not through the cache: the pipelined kernel on a resident
      // grid (measured: dense 1 KiB feature rows 21.1 -> 20.2 us per 65,536
      // ids; for 4 KiB rows, of which a launch gives each wave about two,
      // decode_rows_kernel on a larger grid is as fast or faster, with either
      // pipeline).  With at most 8 invariant bits a stored row is at least
      // about three quarters of its slot, and the pipeline fetches whole
      // slots, 6 workgroups per CU (measured with the Zipf ids: embeddings
      // 12.2 -> 10.2 us, dense features 21.2 -> 18.9 us); otherwise the
      // header window and then the rest of the stream, 8 per CU.
      if constexpr (MODE != kModeCached && NR != 0) {
        if (a.vec && (cd.n == 128 || cd.n == 256 || cd.n == 512)) {
          const bool slot_pipe = cd.p <= kSlotPipeMaxP;
          const uint32_t pipe_grid = row_pipe_grid(cnt, kWavesPerBlock, slot_pipe ? 6u : 8u);
          switch (cd.n) {
            case 128: IBP_PIPE(2); break;
            case 256: IBP_PIPE(4); break;
            default: IBP_PIPE(8); break;
          }
          continue;
        }
      }
      switch (cd.n) {
        case 128: IBP_ROWS(2); break;
        case 256: IBP_ROWS(4); break;
        case 512: IBP_ROWS(8); break;
        case 1024: IBP_ROWS(16); break;
        default: IBP_ROWS(0); break;
      }
#undef IBP_ROWS
#undef IBP_PIPE
    }
    return;
  }
  // segments of kSegBlocks blocks (measured: shorter segments add more
  // header-prefix reads than they gain in parallelism, even for 8 KiB rows)
  const uint64_t seg = small_tasks ? 256 : kSegBlocks;
  const uint32_t nseg = (uint32_t)((cd.n + seg - 1) / seg);
  const uint64_t n_tasks = a.n_out * nseg;
  const uint64_t wgs = (n_tasks + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((decode_segments_kernel<MODE, NR>), dim3(grid_for(wgs)),
                     dim3(kBlockThreads), 0, st, cd, (const uint32_t*)a.slots,
                     (const unsigned long long*)a.flags, a.ids, arena, cloc, a.n_rows, n_tasks,
                     nseg, (uint32_t)seg, (uint32_t*)a.dst, a.vec, (int)a.host_image);
}

template <int MODE>
void launch_decode(const Codec& cd, const DecodeArgs& a, hipStream_t st) {
  switch (cd.runs.n) {
    case 0: launch_decode_t<MODE, 0>(cd, a, st); break;
    case 1: launch_decode_t<MODE, 1>(cd, a, st); break;
    case 2: launch_decode_t<MODE, 2>(cd, a, st); break;
    case 3: launch_decode_t<MODE, 3>(cd, a, st); break;
    case 4: launch_decode_t<MODE, 4>(cd, a, st); break;
    default: launch_decode_t<MODE, -1>(cd, a, st); break;
  }
}

// One launch of compress_pair_wg_kernel over the entries of `b` (rows of
// cd.nw words, 16-bit blocks), sized as launch_compress_wg.
template <int NR>
void launch_compress_pair_wg(const WideCodec<uint16_t>& cd, CompressBatch& b, uint64_t total_rows,
                             hipStream_t st) {
#define IBP_PAIR_WG(CPW, BYTES)                                                             \
  {                                                                                         \
    constexpr uint32_t lds = (CPW * kWave * kWavesPerBlock + 4u + kWavesPerBlock) * 4u;      \
    constexpr uint32_t per_cu = std::min(8u, (160u * 1024u) / lds);                         \
    const uint32_t per_wg =                                                                 \
        cwg_rows_per_wg(total_rows, workgroups_per_device(per_cu), BYTES);                  \
    const uint32_t wgs = set_wg_ends(b, per_wg);                                            \
    hipLaunchKernelGGL((compress_pair_wg_kernel<NR, CPW>), dim3(wgs), dim3(kBlockThreads), 0, \
                       st, cd, b, per_wg);                                                  \
  }
  switch (cd.nw) {
    case 2048: IBP_PAIR_WG(8, true); return;
    case 4096: IBP_PAIR_WG(16, true); return;
    case 7168: IBP_PAIR_WG(28, false); return;
    default: IBP_PAIR_WG(32, false); return;  // 8192
  }
#undef IBP_PAIR_WG
}

// One launch of compress_w64_wg_kernel over the entries of `b` (64-bit blocks
// in rows of 8, 16, 28 or 32 KiB), grid and rows per workgroup as for
// compress_wg_kernel.
template <int NR>
void launch_compress_w64_wg(const WideCodec<uint64_t>& cd, CompressBatch& b,
                            uint64_t total_rows, hipStream_t st) {
#define IBP_W64_WG(CPW, BYTES)                                                              \
  {                                                                                         \
    constexpr uint32_t lds = (2u * CPW * kWave * kWavesPerBlock + 4u + kWavesPerBlock) * 4u; \
    constexpr uint32_t per_cu = std::min(8u, (160u * 1024u) / lds);                         \
    const uint32_t per_wg =                                                                 \
        cwg_rows_per_wg(total_rows, workgroups_per_device(per_cu), BYTES);                  \
    const uint32_t wgs = set_wg_ends(b, per_wg);                                            \
    hipLaunchKernelGGL((compress_w64_wg_kernel<NR, CPW>), dim3(wgs), dim3(kBlockThreads), 0, \
                       st, cd, b, per_wg);                                                  \
  }
  switch (cd.nw) {
    case 2048: IBP_W64_WG(4, true); return;
    case 4096: IBP_W64_WG(8, true); return;
    case 7168: IBP_W64_WG(14, false); return;
    default: IBP_W64_WG(16, false); return;  // 8192
  }
#undef IBP_W64_WG
}

template <typename T, int NR>
void launch_compress_wide_nr(const WideCodec<T>& cd, uint64_t n_rows, const void* src,
                             void* slots, uint64_t* flags, uint32_t* row_bits, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    // rows of 128 * NWL 16-bit blocks (512 bytes to 4 KiB): one wave per row
    const uint64_t wgs = (n_rows + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint32_t grid = (uint32_t)std::min<uint64_t>(wgs, workgroups_per_device(32));
#define IBP_PAIR(NWL)                                                                       \
  hipLaunchKernelGGL((compress_pair_rows_kernel<NR, NWL>), dim3(grid), dim3(kBlockThreads), 0, \
                     st, cd, n_rows, (const uint32_t*)src, (uint32_t*)slots,                 \
                     (unsigned long long*)flags, row_bits)
    switch (cd.nw) {
      case 128: IBP_PAIR(2); return;
      case 256: IBP_PAIR(4); return;
      case 512: IBP_PAIR(8); return;
      case 1024: IBP_PAIR(16); return;
      default: break;
    }
#undef IBP_PAIR
    // rows of 512 * CPW blocks (the 8 and 28 KiB weight rows): a workgroup
    // per row, ranges of rows per workgroup as for compress_wg_kernel
    if (cwg_row(cd.nw)) {
      CompressBatch b{};
      uint64_t total = 0;
      auto flush = [&](CompressBatch& fb, uint64_t rows) {
        launch_compress_pair_wg<NR>(cd, fb, rows, st);
      };
      add_compress_entries(b, total, cd.nw, n_rows, src, slots, flags, row_bits, cd.pad, flush);
      flush(b, total);
      return;
    }
  }
  if constexpr (sizeof(T) == 8) {
    // rows of 64 * NCH 64-bit blocks (512 bytes to 4 KiB): one wave per row
    const uint64_t wgs = (n_rows + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint32_t grid = (uint32_t)std::min<uint64_t>(wgs, workgroups_per_device(32));
#define IBP_W64(NCH)                                                                         \
  hipLaunchKernelGGL((compress_w64_rows_kernel<NR, NCH>), dim3(grid), dim3(kBlockThreads), 0, \
                     st, cd, n_rows, (const uint32_t*)src, (uint32_t*)slots,                  \
                     (unsigned long long*)flags, row_bits)
    switch (cd.nw) {
      case 128: IBP_W64(1); return;
      case 256: IBP_W64(2); return;
      case 512: IBP_W64(4); return;
      case 1024: IBP_W64(8); return;
      default: break;
    }
#undef IBP_W64
    // rows of 256 * CPW blocks (the 8 and 28 KiB weight rows): a workgroup
    // per row, ranges of rows per workgroup as for compress_wg_kernel
    if (cwg_row(cd.nw)) {
      CompressBatch b{};
      uint64_t total = 0;
      auto flush = [&](CompressBatch& fb, uint64_t rows) {
        launch_compress_w64_wg<NR>(cd, fb, rows, st);
      };
      add_compress_entries(b, total, cd.nw, n_rows, src, slots, flags, row_bits, cd.pad, flush);
      flush(b, total);
      return;
    }
  }
#define IBP_WIDE(MAXW)                                                                    \
  hipLaunchKernelGGL((compress_wide_kernel<T, NR, MAXW>), dim3(grid_for(n_rows)),         \
                     dim3(kBlockThreads), 0, st, cd, n_rows, (const uint32_t*)src,         \
                     (uint32_t*)slots, (unsigned long long*)flags, row_bits)
  if (cd.nw <= 1024) IBP_WIDE(1024);
  else if (cd.nw <= 4096) IBP_WIDE(4096);
  else if (cd.nw <= 8192) IBP_WIDE(8192);
  else IBP_WIDE(IBP_MAX_COMPRESS_ROW_BYTES / 4);
#undef IBP_WIDE
}

template <typename T>
void launch_compress_wide(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                          const void* src, void* slots, uint64_t* flags, uint32_t* row_bits,
                          hipStream_t st) {
  WideCodec<T> cd = make_wide_codec<T>(md, row_bytes);
  cd.pad = is_host_memory(slots) ? 0u : 1u;
  switch (cd.nruns) {
    case 0: return launch_compress_wide_nr<T, 0>(cd, n_rows, src, slots, flags, row_bits, st);
    case 1: return launch_compress_wide_nr<T, 1>(cd, n_rows, src, slots, flags, row_bits, st);
    case 2: return launch_compress_wide_nr<T, 2>(cd, n_rows, src, slots, flags, row_bits, st);
    case 3: return launch_compress_wide_nr<T, 3>(cd, n_rows, src, slots, flags, row_bits, st);
    case 4: return launch_compress_wide_nr<T, 4>(cd, n_rows, src, slots, flags, row_bits, st);
    case 5: return launch_compress_wide_nr<T, 5>(cd, n_rows, src, slots, flags, row_bits, st);
    default: return launch_compress_wide_nr<T, -1>(cd, n_rows, src, slots, flags, row_bits, st);
  }
}

template <typename T, int MODE, int NR>
void launch_decode_wide_nr(const WideCodec<T>& cd, const DecodeArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 8 && MODE != kModeCached) {
    // 64-bit blocks in 16-byte aligned rows of 512 bytes to 2 KiB: the row
    // pipeline, in launches of at most 2^30 rows (32-bit row indices)
    if (a.vec && (cd.nw == 128 || cd.nw == 256 || cd.nw == 512)) {
      const uint64_t piece = 1ull << 30;
      for (uint64_t off = 0; off < a.n_out; off += piece) {
        const uint32_t cnt = (uint32_t)std::min<uint64_t>(piece, a.n_out - off);
        const uint32_t* sl = (const uint32_t*)a.slots;
        const unsigned long long* fl = (const unsigned long long*)a.flags;
        if (MODE == kModeTable) {  // flags stay word aligned (piece % 64 == 0)
          sl += off * cd.nw;
          fl += off / 64;
        }
        const int64_t* id_p = MODE != kModeTable ? a.ids + off : a.ids;
        uint32_t* out_p = (uint32_t*)a.dst + off * cd.nw;
        // at most 16 invariant bits of 64 (a stored row is at least about
        // three quarters of its slot): whole slots, as the 32-bit decoder
        // fetches them for p <= 8
        const bool slot_pipe = cd.p <= 2u * kSlotPipeMaxP;
        const uint32_t grid = row_pipe_grid(cnt, kWavesPerBlock, slot_pipe ? 6u : 8u);
#define IBP_P64(NCH, SLOT)                                                                    \
  hipLaunchKernelGGL((decode_pipe64_kernel<MODE, NR, NCH, SLOT>), dim3(grid),                 \
                     dim3(kBlockThreads), 0, st, cd, sl, fl, id_p, a.n_rows, cnt, out_p)
        if (slot_pipe) {
          switch (cd.nw) {
            case 128: IBP_P64(2, true); break;
            case 256: IBP_P64(4, true); break;
            default: IBP_P64(8, true); break;
          }
        } else {
          switch (cd.nw) {
            case 128: IBP_P64(2, false); break;
            case 256: IBP_P64(4, false); break;
            default: IBP_P64(8, false); break;
          }
        }
#undef IBP_P64
      }
      return;
    }
  }
  // a segment's stream stays within the LDS window: <= seg * W / 32 + 3 words
  const uint32_t seg = wide_seg_blocks<T>();
  const uint32_t nseg = (cd.n + seg - 1) / seg;
  const uint64_t n_tasks = a.n_out * nseg;
  const uint64_t wgs = (n_tasks + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((decode_wide_kernel<T, MODE, NR>), dim3(grid_for(wgs)), dim3(kBlockThreads),
                     0, st, cd, (const uint32_t*)a.slots, (const unsigned long long*)a.flags,
                     a.ids, (const uint32_t*)a.arena, (const unsigned long long*)a.cache_loc,
                     a.n_rows, n_tasks, nseg, seg, (T*)a.dst, a.vec, (int)a.host_image);
}

template <typename T, int MODE>
void launch_decode_wide(const ibp_metadata* md, uint64_t row_bytes, const DecodeArgs& a,
                        hipStream_t st) {
  const WideCodec<T> cd = make_wide_codec<T>(md, row_bytes);
  switch (cd.nruns) {
    case 0: return launch_decode_wide_nr<T, MODE, 0>(cd, a, st);
    case 1: return launch_decode_wide_nr<T, MODE, 1>(cd, a, st);
    case 2: return launch_decode_wide_nr<T, MODE, 2>(cd, a, st);
    case 3: return launch_decode_wide_nr<T, MODE, 3>(cd, a, st);
    case 4: return launch_decode_wide_nr<T, MODE, 4>(cd, a, st);
    case 5: return launch_decode_wide_nr<T, MODE, 5>(cd, a, st);
    default: return launch_decode_wide_nr<T, MODE, -1>(cd, a, st);
  }
}

template <typename T>
void launch_decode_wide_mode(const ibp_metadata* md, uint64_t row_bytes, const DecodeArgs& a,
                             int mode, hipStream_t st) {
  if (mode == kModeCached)
    launch_decode_wide<T, kModeCached>(md, row_bytes, a, st);
  else if (mode == kModeGather)
    launch_decode_wide<T, kModeGather>(md, row_bytes, a, st);
  else
    launch_decode_wide<T, kModeTable>(md, row_bytes, a, st);
}

// A batched W = 16 / 64 decode (decode_wide_batch_kernel); n and the slot
// words are per tensor, the rest of the codec is shared.
template <typename T>
void launch_decode_wide_batch(const ibp_metadata* md, const Batch& b, uint32_t grid,
                              uint32_t seg, hipStream_t st) {
  const WideCodec<T> cd = make_wide_codec<T>(md, b.t[0].nw * 4ull);
#define IBP_WBATCH(NR)                                                                      \
  hipLaunchKernelGGL((decode_wide_batch_kernel<T, NR>), dim3(grid), dim3(kBlockThreads), 0, st, \
                     cd, b, seg)
  switch (cd.nruns) {
    case 0: IBP_WBATCH(0); break;
    case 1: IBP_WBATCH(1); break;
    case 2: IBP_WBATCH(2); break;
    case 3: IBP_WBATCH(3); break;
    case 4: IBP_WBATCH(4); break;
    case 5: IBP_WBATCH(5); break;
    default: IBP_WBATCH(-1); break;
  }
#undef IBP_WBATCH
}

// Shift masks for extracting / depositing the bits of `keep` (parallel
// suffix method, Hacker's Delight sections 7-4 and 7-5): step i moves by 2^i
// the kept bits whose count of dropped bits below them has bit i set.
void suffix_masks(uint32_t keep, uint32_t sfx[5]) {
  uint32_t below = ~keep << 1;  // dropped positions, shifted to count "below"
  for (int i = 0; i < 5; ++i) {
    uint32_t par = below ^ (below << 1);  // prefix parity from bit 0 upward
    par ^= par << 2;
    par ^= par << 4;
    par ^= par << 8;
    par ^= par << 16;
    const uint32_t move = par & keep;
    sfx[i] = move;
    keep = (keep ^ move) | (move >> (1u << i));
    below &= ~par;
  }
}

template <uint32_t MAXW>
void launch_compress_positional_t(const void* table, uint32_t n, uint64_t n_rows,
                                  const void* src, void* slots, uint64_t* flags,
                                  uint32_t* row_bits, hipStream_t st) {
  hipLaunchKernelGGL((compress_positional_kernel<MAXW>), dim3(grid_for(n_rows)),
                     dim3(kBlockThreads), 0, st, (const PosEntry*)table, n, n_rows,
                     (const uint32_t*)src, (uint32_t*)slots, (unsigned long long*)flags,
                     row_bits);
}

// Scratch of ibp_build_metadata_noalloc: the count kernel's partial counts
// (up to IBP_NOALLOC_COUNT_GRID workgroups x 64 positions) and the 64
// totals, 513 KiB.  Every device the library runs on holds its own copy
// until the process ends; calls on one device share it.
static __device__ __align__(256) unsigned long long
    scratch[((size_t)IBP_NOALLOC_COUNT_GRID + 1) * 64];
static_assert(IBP_NOALLOC_MAX_WORDS ==
                  (uint64_t)IBP_NOALLOC_COUNT_GRID * kWavesPerBlock * kCountMaxSteps * kCountGroup,
              "the largest no-alloc sample is what IBP_NOALLOC_COUNT_GRID workgroups can count");

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current).  In host code the array's name is
// only a host-side stand-in; kernels get this address instead.
int count_scratch(unsigned long long** out) {
  int rc = pending_hip_error();
  if (rc) return rc;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return IBP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    g_scratch_ptr[dev] = p;
  }
  *out = (unsigned long long*)g_scratch_ptr[dev];
  return IBP_OK;
}

// The tensors of a batch whose rows compress_wg_kernel takes, of one row
// length, in launches of up to kCompressBatchMax entries.
template <int NR>
void compress_wg_batch(const Codec& cd, const ibp_compress_tensor* tensors, uint64_t n_tensors,
                       uint64_t row_bytes, hipStream_t st) {
  CompressBatch b{};
  uint64_t total = 0;
  auto flush = [&](CompressBatch& fb, uint64_t rows) { launch_compress_wg<NR>(cd, fb, rows, st); };
  for (uint64_t t = 0; t < n_tensors; ++t) {
    const ibp_compress_tensor& x = tensors[t];
    if (x.n_rows == 0 || x.row_bytes != row_bytes) continue;
    add_compress_entries(b, total, cd.n, x.n_rows, x.src, x.slots, x.flags, x.row_bits,
                         is_host_memory(x.slots) ? 0u : 1u, flush);
  }
  if (b.count) flush(b, total);
}

// The same for 16-bit blocks and compress_pair_wg_kernel.
template <int NR>
void compress_pair_batch(const WideCodec<uint16_t>& cd, const ibp_compress_tensor* tensors,
                         uint64_t n_tensors, uint64_t row_bytes, hipStream_t st) {
  CompressBatch b{};
  uint64_t total = 0;
  auto flush = [&](CompressBatch& fb, uint64_t rows) {
    launch_compress_pair_wg<NR>(cd, fb, rows, st);
  };
  for (uint64_t t = 0; t < n_tensors; ++t) {
    const ibp_compress_tensor& x = tensors[t];
    if (x.n_rows == 0 || x.row_bytes != row_bytes) continue;
    add_compress_entries(b, total, cd.nw, x.n_rows, x.src, x.slots, x.flags, x.row_bits,
                         is_host_memory(x.slots) ? 0u : 1u, flush);
  }
  if (b.count) flush(b, total);
}

template <int NR>
void compress_w64_batch(const WideCodec<uint64_t>& cd, const ibp_compress_tensor* tensors,
                        uint64_t n_tensors, uint64_t row_bytes, hipStream_t st) {
  CompressBatch b{};
  uint64_t total = 0;
  auto flush = [&](CompressBatch& fb, uint64_t rows) {
    launch_compress_w64_wg<NR>(cd, fb, rows, st);
  };
  for (uint64_t t = 0; t < n_tensors; ++t) {
    const ibp_compress_tensor& x = tensors[t];
    if (x.n_rows == 0 || x.row_bytes != row_bytes) continue;
    add_compress_entries(b, total, cd.nw, x.n_rows, x.src, x.slots, x.flags, x.row_bits,
                         is_host_memory(x.slots) ? 0u : 1u, flush);
  }
  if (b.count) flush(b, total);
}

}  // namespace

// ------------------------------------------------------------ C ABI ----

extern "C" {

uint64_t ibp_flag_words(uint64_t n_rows) { return n_rows / 64 + (n_rows % 64 ? 1 : 0); }

int ibp_last_hip_error(void) { return g_last_hip; }

const char* ibp_status_string(int status) {
  switch (status) {
    case IBP_OK: return "ok";
    case IBP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case IBP_ERR_UNSUPPORTED: return "unsupported block width or row size";
    case IBP_ERR_LAYOUT: return "bad layout (row_bytes not a multiple of 4, or misaligned pointer)";
    case IBP_ERR_EMPTY: return "empty sample";
    case IBP_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int ibp_metadata_from_counts(const uint64_t* ones, uint64_t n_blocks, uint32_t width_bits,
                             uint32_t t_ppm, ibp_metadata* out) {
  if (!ones || !out || t_ppm > 1000000u) return IBP_ERR_INVALID_ARGUMENT;
  if (!width_supported(width_bits)) return IBP_ERR_UNSUPPORTED;
  if (n_blocks == 0) return IBP_ERR_EMPTY;
  uint64_t mask = 0, bitval = 0;
  for (uint32_t b = 0; b < width_bits; ++b) {
    if (ones[b] > n_blocks) return IBP_ERR_INVALID_ARGUMENT;
    const uint64_t zeros = n_blocks - ones[b];
    const bool one_wins = ones[b] > zeros;  // a tie records 0
    const unsigned __int128 count = one_wins ? ones[b] : zeros;
    if (count * 1000000u >= (unsigned __int128)n_blocks * t_ppm) {
      mask |= 1ull << b;
      if (one_wins) bitval |= 1ull << b;
    }
  }
  out->width_bits = width_bits;
  out->invariant_bits = (uint32_t)popcount32(mask);
  out->mask = mask;
  out->bitval = bitval;
  out->t_ppm = t_ppm;
  out->reserved = 0;
  return IBP_OK;
}

// [IBP] Preprocessing on the GPU.  scratch: device buffer of at least
// (grid + 1) * 64 counters for the count kernel's partials and the totals,
// with grid <= max_grid; nullptr: allocate one for the call.
static int build_metadata_impl(const void* sample, uint64_t n_blocks, uint32_t width_bits,
                               uint32_t t_ppm, ibp_metadata* out, uint64_t* out_ones,
                               void* stream, unsigned long long* scratch, uint64_t max_grid) {
  if (!sample || !out || t_ppm > 1000000u) return IBP_ERR_INVALID_ARGUMENT;
  if (!width_supported(width_bits)) return IBP_ERR_UNSUPPORTED;
  if (n_blocks == 0) return IBP_ERR_EMPTY;
  if (n_blocks > (1ull << 56)) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(sample, 4)) return IBP_ERR_LAYOUT;
  hipStream_t st = (hipStream_t)stream;
  // The kernel counts 32-bit words: W = 16 adds the two halves of every word
  // (and a last odd block on the host), W = 64 counts even and odd words.
  const uint64_t words = width_bits == 16 ? n_blocks / 2
                         : width_bits == 32 ? n_blocks : 2 * n_blocks;
  const int npos = width_bits == 64 ? 64 : 32;
  uint64_t counts[64] = {0};
  uint16_t odd_block = 0;
  hipError_t e = hipSuccess;
  unsigned long long* d_buf = nullptr;
  if (words) {
    // about two workgroups per CU; more only when a wave would otherwise take
    // more than kCountMaxSteps steps (its lanes' counts must stay below 2^24)
    const uint64_t steps = (words + kCountGroup - 1) / kCountGroup;
    uint64_t wgs = std::min<uint64_t>((steps + kWavesPerBlock - 1) / kWavesPerBlock,
                                      workgroups_per_device(2));
    if (scratch) wgs = std::min<uint64_t>(wgs, max_grid);
    const uint64_t per_wg = kCountMaxSteps * kWavesPerBlock;
    wgs = std::max<uint64_t>({wgs, (steps + per_wg - 1) / per_wg, 1});
    if (wgs > kMaxGrid) return IBP_ERR_INVALID_ARGUMENT;
    if (scratch && wgs > max_grid) return IBP_ERR_UNSUPPORTED;  // sample too large
    const uint32_t grid = (uint32_t)wgs;
    const uint64_t lane_max =
        (steps + wgs * kWavesPerBlock - 1) / (wgs * kWavesPerBlock) * kCountWords;
    int rc = pending_hip_error();
    if (rc) return rc;
    // partial counts (npos columns of grid) followed by the npos totals
    if (scratch) {
      d_buf = scratch;
    } else {
      e = hipMalloc((void**)&d_buf, ((size_t)grid + 1) * npos * sizeof(unsigned long long));
      if (e != hipSuccess) return hip_fail(e);
    }
    unsigned long long* d_counts = d_buf + (size_t)grid * npos;
    const uint32_t* smp = (const uint32_t*)sample;
#define IBP_COUNT(P, NPOS)                                                              \
  hipLaunchKernelGGL((count_ones_kernel<P, NPOS>), dim3(grid), dim3(kBlockThreads), 0, st, \
                     smp, words, d_buf)
#define IBP_COUNT_NPOS(NPOS)                     \
  if (lane_max < (1u << 8)) IBP_COUNT(8, NPOS);  \
  else if (lane_max < (1u << 12)) IBP_COUNT(12, NPOS); \
  else if (lane_max < (1u << 16)) IBP_COUNT(16, NPOS); \
  else IBP_COUNT(24, NPOS);
    if (npos == 64) {
      IBP_COUNT_NPOS(64)
    } else {
      IBP_COUNT_NPOS(32)
    }
#undef IBP_COUNT_NPOS
#undef IBP_COUNT
    hipLaunchKernelGGL(reduce_counts_kernel, dim3(npos / kWavesPerBlock), dim3(kBlockThreads), 0,
                       st, (const unsigned long long*)d_buf, grid, d_counts);
    e = hipGetLastError();
    if (e == hipSuccess)
      e = hipMemcpyAsync(counts, d_counts, npos * sizeof(uint64_t), hipMemcpyDeviceToHost, st);
  } else {
    int rc = pending_hip_error();
    if (rc) return rc;
  }
  if (e == hipSuccess && width_bits == 16 && (n_blocks & 1))
    e = hipMemcpyAsync(&odd_block, (const uint16_t*)sample + (n_blocks - 1), 2,
                       hipMemcpyDefault, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (d_buf && !scratch) {
    hipError_t ef = hipFree(d_buf);
    if (e == hipSuccess) e = ef;
  }
  if (e != hipSuccess) return hip_fail(e);
  uint64_t ones[64];
  for (uint32_t b = 0; b < width_bits; ++b)
    ones[b] = width_bits == 16 ? counts[b] + counts[b + 16] + ((odd_block >> b) & 1u) : counts[b];
  if (out_ones)
    for (uint32_t b = 0; b < width_bits; ++b) out_ones[b] = ones[b];
  return ibp_metadata_from_counts(ones, n_blocks, width_bits, t_ppm, out);
}

int ibp_build_metadata(const void* sample, uint64_t n_blocks, uint32_t width_bits,
                       uint32_t t_ppm, ibp_metadata* out, uint64_t* out_ones,
                       void* stream) {
  return build_metadata_impl(sample, n_blocks, width_bits, t_ppm, out, out_ones, stream,
                             nullptr, 0);
}

int ibp_build_metadata_noalloc(const void* sample, uint64_t n_blocks, uint32_t width_bits,
                               uint32_t t_ppm, ibp_metadata* out, uint64_t* out_ones,
                               void* stream) {
  // argument errors first, as ibp_build_metadata reports them
  if (!sample || !out || t_ppm > 1000000u) return IBP_ERR_INVALID_ARGUMENT;
  if (!width_supported(width_bits)) return IBP_ERR_UNSUPPORTED;
  if (n_blocks == 0) return IBP_ERR_EMPTY;
  unsigned long long* buf = nullptr;
  const int rc = count_scratch(&buf);
  if (rc) return rc;
  return build_metadata_impl(sample, n_blocks, width_bits, t_ppm, out, out_ones, stream, buf,
                             IBP_NOALLOC_COUNT_GRID);
}

// Host checks of ibp_compress's arguments (n_rows == 0 passes).
static int check_compress(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                          const void* src, const void* slots, const uint64_t* flags,
                          const uint32_t* row_bits) {
  int rc = check_rows(n_rows, row_bytes, md->width_bits);
  if (rc) return rc;
  if (row_bytes > IBP_MAX_COMPRESS_ROW_BYTES) return IBP_ERR_UNSUPPORTED;
  if (n_rows == 0) return IBP_OK;
  if (!src || !slots || !flags) return IBP_ERR_INVALID_ARGUMENT;
  const uintptr_t al = md->width_bits == 64 ? 8 : 4;
  if (!aligned(src, al) || !aligned(slots, al) || !aligned(flags, 8) ||
      (row_bits && !aligned(row_bits, 4)))
    return IBP_ERR_LAYOUT;
  {  // in place (src == slots) is allowed, any other overlap is not
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)slots, len = n_rows * row_bytes;
    if (a != b && a < b + len && b < a + len) return IBP_ERR_INVALID_ARGUMENT;
  }
  return IBP_OK;
}

// Enqueues the compression of one checked tensor (n_rows > 0).
static void enqueue_compress(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                             const void* src, void* slots, uint64_t* flags, uint32_t* row_bits,
                             hipStream_t st) {
  // no clearing launch: every row's flag bit is cleared or set by the
  // kernel that compresses the row
  if (md->width_bits != 32) {
    if (md->width_bits == 16)
      launch_compress_wide<uint16_t>(md, n_rows, row_bytes, src, slots, flags, row_bits, st);
    else
      launch_compress_wide<uint64_t>(md, n_rows, row_bytes, src, slots, flags, row_bits, st);
    return;
  }
  Codec cd = make_codec(md, row_bytes);
  cd.pad = is_host_memory(slots) ? 0u : 1u;
  const int vec = row_bytes % 16 == 0 && aligned(src, 16) && aligned(slots, 16);
  switch (cd.runs.n) {
    case 0: launch_compress_nr<0>(cd, n_rows, src, slots, flags, row_bits, vec, st); break;
    case 1: launch_compress_nr<1>(cd, n_rows, src, slots, flags, row_bits, vec, st); break;
    case 2: launch_compress_nr<2>(cd, n_rows, src, slots, flags, row_bits, vec, st); break;
    case 3: launch_compress_nr<3>(cd, n_rows, src, slots, flags, row_bits, vec, st); break;
    case 4: launch_compress_nr<4>(cd, n_rows, src, slots, flags, row_bits, vec, st); break;
    default: launch_compress_nr<-1>(cd, n_rows, src, slots, flags, row_bits, vec, st); break;
  }
}

int ibp_compress(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes, const void* src,
                 void* slots, uint64_t* flags, uint32_t* row_bits, void* stream) {
  int rc = check_metadata(md);
  if (rc) return rc;
  rc = check_compress(md, n_rows, row_bytes, src, slots, flags, row_bits);
  if (rc || n_rows == 0) return rc;
  rc = pending_hip_error();
  if (rc) return rc;
  enqueue_compress(md, n_rows, row_bytes, src, slots, flags, row_bits, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

int ibp_compress_batch(const ibp_metadata* md, const ibp_compress_tensor* tensors,
                       uint64_t n_tensors, void* stream) {
  int rc = check_metadata(md);
  if (rc) return rc;
  if (n_tensors == 0) return IBP_OK;
  if (!tensors) return IBP_ERR_INVALID_ARGUMENT;
  bool work = false;
  for (uint64_t t = 0; t < n_tensors; ++t) {
    const ibp_compress_tensor& x = tensors[t];
    rc = check_compress(md, x.n_rows, x.row_bytes, x.src, x.slots, x.flags, x.row_bits);
    if (rc) return rc;
    work = work || x.n_rows != 0;
  }
  if (!work) return IBP_OK;
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  bool done[4] = {false, false, false, false};  // the four row lengths of cwg_row
  for (uint64_t t = 0; t < n_tensors; ++t) {
    const ibp_compress_tensor& x = tensors[t];
    if (x.n_rows == 0) continue;
    const uint64_t n = x.row_bytes / 4;  // words of a row
    if (!cwg_row((uint32_t)n)) {  // tensor by tensor
      enqueue_compress(md, x.n_rows, x.row_bytes, x.src, x.slots, x.flags, x.row_bits, st);
      continue;
    }
    // the first tensor of each row length of the weight-row kernels gathers
    // every tensor of that length into shared launches
    bool& d = done[n == 2048 ? 0 : n == 4096 ? 1 : n == 7168 ? 2 : 3];
    if (d) continue;
    d = true;
    if (md->width_bits == 32) {
      const Codec cd = make_codec(md, x.row_bytes);
      switch (cd.runs.n) {
        case 0: compress_wg_batch<0>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 1: compress_wg_batch<1>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 2: compress_wg_batch<2>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 3: compress_wg_batch<3>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 4: compress_wg_batch<4>(cd, tensors, n_tensors, x.row_bytes, st); break;
        default: compress_wg_batch<-1>(cd, tensors, n_tensors, x.row_bytes, st); break;
      }
    } else if (md->width_bits == 64) {
      const WideCodec<uint64_t> cd = make_wide_codec<uint64_t>(md, x.row_bytes);
      switch (cd.nruns) {
        case 0: compress_w64_batch<0>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 1: compress_w64_batch<1>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 2: compress_w64_batch<2>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 3: compress_w64_batch<3>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 4: compress_w64_batch<4>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 5: compress_w64_batch<5>(cd, tensors, n_tensors, x.row_bytes, st); break;
        default: compress_w64_batch<-1>(cd, tensors, n_tensors, x.row_bytes, st); break;
      }
    } else {
      const WideCodec<uint16_t> cd = make_wide_codec<uint16_t>(md, x.row_bytes);
      switch (cd.nruns) {
        case 0: compress_pair_batch<0>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 1: compress_pair_batch<1>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 2: compress_pair_batch<2>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 3: compress_pair_batch<3>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 4: compress_pair_batch<4>(cd, tensors, n_tensors, x.row_bytes, st); break;
        case 5: compress_pair_batch<5>(cd, tensors, n_tensors, x.row_bytes, st); break;
        default: compress_pair_batch<-1>(cd, tensors, n_tensors, x.row_bytes, st); break;
      }
    }
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

static int decode_common(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                         const void* slots, const uint64_t* flags, const int64_t* ids,
                         uint64_t n_out, void* dst, void* stream, int mode,
                         const void* arena = nullptr, const uint64_t* cache_loc = nullptr) {
  int rc = check_metadata(md);
  if (rc) return rc;
  rc = check_rows(n_rows, row_bytes, md->width_bits);
  if (rc) return rc;
  if (n_out > UINT64_MAX / row_bytes) return IBP_ERR_INVALID_ARGUMENT;
  if (n_out == 0) return IBP_OK;
  const bool gather = mode != kModeTable;
  if (n_rows == 0 || !slots || !flags || !dst || (gather && !ids))
    return IBP_ERR_INVALID_ARGUMENT;
  if (mode == kModeCached && (!arena || !cache_loc)) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(slots, 4) || !aligned(dst, 4) || !aligned(flags, 8) ||
      (gather && !aligned(ids, 8)))
    return IBP_ERR_LAYOUT;
  if (mode == kModeCached && (!aligned(arena, 16) || !aligned(cache_loc, 8)))
    return IBP_ERR_LAYOUT;
  if (md->width_bits == 64 && (!aligned(slots, 8) || !aligned(dst, 8))) return IBP_ERR_LAYOUT;
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (md->width_bits != 32) {
    // 16-byte staging and raw copies need 16-byte rows (segments are
    // multiples of 64 blocks, so their bounds are 16-byte aligned too)
    const int vec = row_bytes % 16 == 0 && aligned(slots, 16) && aligned(dst, 16);
    const DecodeArgs a{slots, flags, ids, arena, cache_loc, n_rows, n_out, dst, vec,
                       is_host_memory(slots)};
    if (md->width_bits == 16)
      launch_decode_wide_mode<uint16_t>(md, row_bytes, a, mode, st);
    else
      launch_decode_wide_mode<uint64_t>(md, row_bytes, a, mode, st);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? IBP_OK : hip_fail(e);
  }
  const Codec cd = make_codec(md, row_bytes);
  // cache entries start at 16-byte boundaries of the (16-byte aligned) arena
  const int vec = row_bytes % 16 == 0 && aligned(slots, 16) && aligned(dst, 16);
  const DecodeArgs a{slots, flags, ids, arena, cache_loc, n_rows, n_out, dst, vec,
                     is_host_memory(slots)};
  if (mode == kModeCached)
    launch_decode<kModeCached>(cd, a, st);
  else if (gather)
    launch_decode<kModeGather>(cd, a, st);
  else
    launch_decode<kModeTable>(cd, a, st);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

int ibp_decompress(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                   const void* slots, const uint64_t* flags, void* dst, void* stream) {
  return decode_common(md, n_rows, row_bytes, slots, flags, nullptr, n_rows, dst, stream,
                       kModeTable);
}

// Blocks per task of a batched decode: a segment's stream stays within the
// LDS window (<= seg * W / 32 + 3 words).
static uint32_t batch_seg(uint32_t width_bits) {
  return width_bits == 64 ? wide_seg_blocks<uint64_t>()
                          : width_bits == 16 ? wide_seg_blocks<uint16_t>() : kSegBlocks;
}

// Host checks of one tensor of a batch (those of decode_common for a full
// decompress).
static int check_batch_tensor(const ibp_metadata* md, const ibp_tensor& t) {
  int rc = check_rows(t.n_rows, t.row_bytes, md->width_bits);
  if (rc) return rc;
  if (t.n_rows == 0) return IBP_OK;
  if (!t.slots || !t.flags || !t.dst) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(t.slots, 4) || !aligned(t.dst, 4) || !aligned(t.flags, 8)) return IBP_ERR_LAYOUT;
  if (md->width_bits == 64 && (!aligned(t.slots, 8) || !aligned(t.dst, 8))) return IBP_ERR_LAYOUT;
  // task counts of the batched launch fit their 56 bits
  const uint64_t nseg = (t.row_bytes * 8 / md->width_bits + batch_seg(md->width_bits) - 1) /
                        batch_seg(md->width_bits);
  if (t.n_rows > (UINT64_MAX >> 8) / nseg) return IBP_ERR_INVALID_ARGUMENT;
  return IBP_OK;
}

int ibp_decompress_batch(const ibp_metadata* md, const ibp_tensor* tensors, uint64_t n_tensors,
                         void* stream) {
  int rc = check_metadata(md);
  if (rc) return rc;
  if (n_tensors == 0) return IBP_OK;
  if (!tensors) return IBP_ERR_INVALID_ARGUMENT;
  bool work = false;
  for (uint64_t t = 0; t < n_tensors; ++t) {
    rc = check_batch_tensor(md, tensors[t]);
    if (rc) return rc;
    work = work || tensors[t].n_rows != 0;
  }
  if (!work) return IBP_OK;
  rc = pending_hip_error();
  if (rc) return rc;
  const uint32_t W = md->width_bits;
  if (W == 64) {  // rows of 512 B to 2 KiB decode faster through the row pipeline
    bool pipe = false;
    for (uint64_t t = 0; t < n_tensors; ++t) {
      const uint64_t rb = tensors[t].row_bytes;
      pipe = pipe || (tensors[t].n_rows && (rb == 512 || rb == 1024 || rb == 2048));
    }
    if (pipe) {  // tensor by tensor
      for (uint64_t t = 0; t < n_tensors; ++t) {
        const ibp_tensor& x = tensors[t];
        if (x.n_rows == 0) continue;
        rc = ibp_decompress(md, x.n_rows, x.row_bytes, x.slots, x.flags, x.dst, stream);
        if (rc) return rc;
      }
      return IBP_OK;
    }
  }
  hipStream_t st = (hipStream_t)stream;
  const uint32_t seg = batch_seg(W);
  uint64_t t = 0;
  while (t < n_tensors) {
    Batch b{};
    uint64_t tasks = 0;
    for (; t < n_tensors && b.count < kBatchMax; ++t) {
      const ibp_tensor& x = tensors[t];
      if (x.n_rows == 0) continue;
      const uint32_t n = (uint32_t)(x.row_bytes * 8 / W);
      const uint32_t nseg = (n + seg - 1) / seg;  // checked above
      tasks += x.n_rows * nseg;
      BatchTensor& bt = b.t[b.count];
      bt.slots = (const uint32_t*)x.slots;
      bt.flags = (const unsigned long long*)x.flags;
      bt.dst = (uint32_t*)x.dst;
      bt.n = n;
      bt.nseg = nseg;
      bt.vec = x.row_bytes % 16 == 0 && aligned(x.slots, 16) && aligned(x.dst, 16);
      bt.nw = (uint32_t)(x.row_bytes / 4);
      b.end[b.count] = tasks;
      ++b.count;
    }
    if (b.count == 0) break;
    const uint32_t grid = grid_for((tasks + kWavesPerBlock - 1) / kWavesPerBlock);
    if (W == 32) {
      const Codec cd = make_codec(md, tensors[0].row_bytes);  // n is per tensor
#define IBP_BATCH(NR)                                                                      \
  hipLaunchKernelGGL((decode_batch_kernel<NR>), dim3(grid), dim3(kBlockThreads), 0, st, cd, b)
      switch (cd.runs.n) {
        case 0: IBP_BATCH(0); break;
        case 1: IBP_BATCH(1); break;
        case 2: IBP_BATCH(2); break;
        case 3: IBP_BATCH(3); break;
        case 4: IBP_BATCH(4); break;
        default: IBP_BATCH(-1); break;
      }
#undef IBP_BATCH
    } else if (W == 16) {
      launch_decode_wide_batch<uint16_t>(md, b, grid, seg, st);
    } else {
      launch_decode_wide_batch<uint64_t>(md, b, grid, seg, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  return IBP_OK;
}

int ibp_gather_decompress(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                          const void* slots, const uint64_t* flags, const int64_t* row_ids,
                          uint64_t n_ids, void* dst, void* stream) {
  return decode_common(md, n_rows, row_bytes, slots, flags, row_ids, n_ids, dst, stream,
                       kModeGather);
}

static int check_cache_image(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                             const void* slots, const uint64_t* flags, const int64_t* row_ids,
                             uint64_t n_ids) {
  int rc = check_metadata(md);
  if (rc) return rc;
  rc = check_rows(n_rows, row_bytes, md->width_bits);
  if (rc) return rc;
  if (n_ids > (1ull << 36)) return IBP_ERR_INVALID_ARGUMENT;  // scan tiles fit one grid
  if (n_ids == 0) return IBP_OK;
  if (n_rows == 0 || !slots || !flags || !row_ids) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(slots, 4) || !aligned(flags, 8) || !aligned(row_ids, 8)) return IBP_ERR_LAYOUT;
  return IBP_OK;
}

int ibp_cache_plan(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                   const void* slots, const uint64_t* flags, const int64_t* row_ids,
                   uint64_t n_ids, uint64_t* entry_loc, uint64_t* arena_bytes, void* stream) {
  int rc = check_cache_image(md, n_rows, row_bytes, slots, flags, row_ids, n_ids);
  if (rc) return rc;
  if (!arena_bytes) return IBP_ERR_INVALID_ARGUMENT;
  if (n_ids == 0) {
    *arena_bytes = 0;
    return IBP_OK;
  }
  if (!entry_loc) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(entry_loc, 8)) return IBP_ERR_LAYOUT;
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const uint64_t n_tiles = (n_ids + kScanTile - 1) / kScanTile;  // <= 2^24
  unsigned long long* d_sums = nullptr;
  hipError_t e = hipMalloc((void**)&d_sums, (n_tiles + 1) * sizeof(unsigned long long));
  if (e != hipSuccess) return hip_fail(e);
  unsigned long long* loc = (unsigned long long*)entry_loc;
  const uint64_t size_wgs = (n_ids + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(cache_sizes_kernel,
                     dim3((uint32_t)std::min<uint64_t>(size_wgs, workgroups_per_device(16))),
                     dim3(kBlockThreads), 0, st, (uint32_t)(row_bytes * 8 / md->width_bits),
                     (uint32_t)(row_bytes / 4), md->width_bits, md->invariant_bits,
                     (const uint32_t*)slots, (const unsigned long long*)flags, row_ids, n_rows,
                     n_ids, loc);
  hipLaunchKernelGGL(cache_tile_sums_kernel, dim3((uint32_t)n_tiles), dim3(kBlockThreads), 0, st,
                     (const unsigned long long*)loc, n_ids, d_sums);
  hipLaunchKernelGGL(cache_scan_sums_kernel, dim3(1), dim3(kBlockThreads), 0, st, d_sums,
                     (uint32_t)n_tiles);
  hipLaunchKernelGGL(cache_offsets_kernel, dim3((uint32_t)n_tiles), dim3(kBlockThreads), 0, st,
                     loc, n_ids, (const unsigned long long*)d_sums);
  unsigned long long units = 0;
  e = hipGetLastError();
  if (e == hipSuccess)
    e = hipMemcpyAsync(&units, d_sums + n_tiles, sizeof(units), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  hipError_t ef = hipFree(d_sums);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return hip_fail(e);
  if (units > IBP_LOC_OFFSET_MASK) return IBP_ERR_UNSUPPORTED;
  *arena_bytes = units * 16;
  return IBP_OK;
}

int ibp_cache_fill(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                   const void* slots, const uint64_t* flags, const int64_t* row_ids,
                   uint64_t n_ids, const uint64_t* entry_loc, void* arena,
                   uint64_t arena_bytes, uint64_t* cache_loc, void* stream) {
  int rc = check_cache_image(md, n_rows, row_bytes, slots, flags, row_ids, n_ids);
  if (rc) return rc;
  if (!cache_loc || (n_ids && (!entry_loc || (!arena && arena_bytes))))
    return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(cache_loc, 8) || (entry_loc && !aligned(entry_loc, 8)) ||
      (arena && !aligned(arena, 16)))
    return IBP_ERR_LAYOUT;
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_for((n_rows + 255) / 256)), dim3(256), 0, st,
                     (unsigned long long*)cache_loc, n_rows, 0ull);
  if (n_ids && arena_bytes >= 16) {
    const uint64_t wgs = (n_ids + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(cache_fill_kernel,
                       dim3((uint32_t)std::min<uint64_t>(wgs, workgroups_per_device(16))),
                       dim3(kBlockThreads), 0, st, (uint32_t)(row_bytes / 4),
                       (const uint32_t*)slots, row_ids, (const unsigned long long*)entry_loc,
                       n_ids, n_rows, (uint32_t*)arena, arena_bytes / 16,
                       (unsigned long long*)cache_loc);
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

int ibp_gather_decompress_cached(const ibp_metadata* md, uint64_t n_rows, uint64_t row_bytes,
                                 const void* arena, const uint64_t* cache_loc,
                                 const void* slots, const uint64_t* flags,
                                 const int64_t* row_ids, uint64_t n_ids, void* dst,
                                 void* stream) {
  return decode_common(md, n_rows, row_bytes, slots, flags, row_ids, n_ids, dst, stream,
                       kModeCached, arena, cache_loc);
}

uint64_t ibp_positional_table_bytes(uint64_t n_positions) {
  return n_positions * sizeof(PosEntry) + (n_positions + 63) / 64 * kPlaneWords * 8;
}

int ibp_positional_table(const uint32_t* mask, const uint32_t* bitval, uint64_t n_positions,
                         void* table) {
  if (n_positions && (!mask || !bitval || !table)) return IBP_ERR_INVALID_ARGUMENT;
  if (n_positions > (1ull << 24)) return IBP_ERR_INVALID_ARGUMENT;
  for (uint64_t k = 0; k < n_positions; ++k)
    if (bitval[k] & ~mask[k]) return IBP_ERR_INVALID_ARGUMENT;
  PosEntry* e = (PosEntry*)table;
  unsigned long long* planes = (unsigned long long*)(e + n_positions);
  const uint64_t n_chunks = (n_positions + 63) / 64;
  for (uint64_t i = 0; i < n_chunks * kPlaneWords; ++i) planes[i] = 0;
  for (uint64_t k = 0; k < n_positions; ++k) {
    e[k].mask = mask[k];
    e[k].bitval = bitval[k];
    e[k].p = (uint32_t)popcount32(mask[k]);
    suffix_masks(~mask[k], e[k].sfx);
    for (int t = 0; t < 6; ++t)
      if ((e[k].p >> t) & 1u) planes[(k / 64) * kPlaneWords + t] |= 1ull << (k % 64);
  }
  return IBP_OK;
}

int ibp_build_metadata_positional(const void* sample, uint64_t n_sample_rows,
                                  uint64_t row_bytes, uint32_t t_ppm, void* table,
                                  uint32_t* mask_out, uint32_t* bitval_out, void* stream) {
  if (!sample || !table || t_ppm > 1000000u) return IBP_ERR_INVALID_ARGUMENT;
  int rc = check_rows(n_sample_rows, row_bytes);
  if (rc) return rc;
  if (n_sample_rows == 0) return IBP_ERR_EMPTY;
  if (n_sample_rows >= (1ull << 32) || row_bytes / 4 > (1u << 24)) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(sample, 4) || !aligned(table, 16)) return IBP_ERR_LAYOUT;
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const uint32_t n = (uint32_t)(row_bytes / 4);
  const uint32_t n_chunks = (n + kWave - 1) / kWave;
  // rows per wave task: a multiple of 32 below 2^12, enough tasks to fill the GPU
  uint64_t rows_per_task =
      (n_sample_rows * n_chunks + (uint64_t)workgroups_per_device(8) * kWavesPerBlock - 1) /
      ((uint64_t)workgroups_per_device(8) * kWavesPerBlock);
  rows_per_task = std::min<uint64_t>(2048, std::max<uint64_t>(32, (rows_per_task + 31) / 32 * 32));
  const uint64_t n_ranges = (n_sample_rows + rows_per_task - 1) / rows_per_task;
  const uint64_t n_tasks = n_ranges * n_chunks;
  const uint64_t wgs = (n_tasks + kWavesPerBlock - 1) / kWavesPerBlock;
  if (wgs > kMaxGrid) return IBP_ERR_INVALID_ARGUMENT;
  uint32_t* d_counts = nullptr;
  hipError_t e = hipMalloc((void**)&d_counts, (size_t)n * 32 * sizeof(uint32_t));
  if (e != hipSuccess) return hip_fail(e);
  hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_for(((uint64_t)n * 16 + 255) / 256)), dim3(256),
                     0, st, (unsigned long long*)d_counts, (uint64_t)n * 16, 0ull);
  hipLaunchKernelGGL(count_positions_kernel, dim3((uint32_t)wgs), dim3(kBlockThreads), 0, st,
                     (const uint32_t*)sample, n_sample_rows, n, n_chunks,
                     (uint32_t)rows_per_task, n_tasks, d_counts);
  std::vector<uint32_t> counts((size_t)n * 32);
  e = hipGetLastError();
  if (e == hipSuccess)
    e = hipMemcpyAsync(counts.data(), d_counts, counts.size() * sizeof(uint32_t),
                       hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  hipError_t ef = hipFree(d_counts);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return hip_fail(e);
  std::vector<uint32_t> mask(n), bitval(n);
  for (uint32_t k = 0; k < n; ++k) {
    uint64_t ones[32];
    for (int b = 0; b < 32; ++b) ones[b] = counts[(size_t)k * 32 + b];
    ibp_metadata md;
    rc = ibp_metadata_from_counts(ones, n_sample_rows, 32, t_ppm, &md);
    if (rc) return rc;
    mask[k] = (uint32_t)md.mask;
    bitval[k] = (uint32_t)md.bitval;
  }
  std::vector<unsigned char> host(ibp_positional_table_bytes(n));
  rc = ibp_positional_table(mask.data(), bitval.data(), n, host.data());
  if (rc) return rc;
  e = hipMemcpyAsync(table, host.data(), host.size(), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e);
  if (mask_out)
    for (uint32_t k = 0; k < n; ++k) mask_out[k] = mask[k];
  if (bitval_out)
    for (uint32_t k = 0; k < n; ++k) bitval_out[k] = bitval[k];
  return IBP_OK;
}

int ibp_compress_positional(const void* table, uint64_t n_rows, uint64_t row_bytes,
                            const void* src, void* slots, uint64_t* flags, uint32_t* row_bits,
                            void* stream) {
  if (!table) return IBP_ERR_INVALID_ARGUMENT;
  int rc = check_rows(n_rows, row_bytes);
  if (rc) return rc;
  if (row_bytes > IBP_MAX_COMPRESS_ROW_BYTES) return IBP_ERR_UNSUPPORTED;
  if (n_rows == 0) return IBP_OK;
  if (!src || !slots || !flags) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(table, 16) || !aligned(src, 4) || !aligned(slots, 4) || !aligned(flags, 8) ||
      (row_bits && !aligned(row_bits, 4)))
    return IBP_ERR_LAYOUT;
  {  // in place (src == slots) is allowed, any other overlap is not
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)slots, len = n_rows * row_bytes;
    if (a != b && a < b + len && b < a + len) return IBP_ERR_INVALID_ARGUMENT;
  }
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  // no clearing launch: every row's flag bit is cleared or set by the
  // kernel that compresses the row (put_flag_bits)
  const uint32_t n = (uint32_t)(row_bytes / 4);
  if (n == 128 || n == 256 || n == 512 || n == 1024) {
    // one wave per row, the table in LDS per workgroup; four times as many
    // workgroups as stay resident (two for rows of 1024 blocks, whose 28 KiB
    // table is costlier to stage), so the dispatcher balances the row ranges:
    // per-position embeddings 1.17 -> 1.10 ms, dense features 1.07 -> 0.99 ms
    // against a resident grid
    const uint32_t pad = is_host_memory(slots) ? 0u : 1u;
#define IBP_CPR(NCH, WPB, PER_CU)                                                              \
  hipLaunchKernelGGL((compress_pos_rows_kernel<NCH, WPB>),                                     \
                     dim3((uint32_t)std::min<uint64_t>((n_rows + WPB - 1) / WPB,               \
                                                       workgroups_per_device(PER_CU))),        \
                     dim3(WPB * kWave), 0, st, (const PosEntry*)table, n_rows,                 \
                     (const uint32_t*)src, (uint32_t*)slots, (unsigned long long*)flags,       \
                     row_bits, pad)
    switch (n) {
      case 128: IBP_CPR(2, 4, 32); break;
      case 256: IBP_CPR(4, 4, 32); break;
      case 512: IBP_CPR(8, 4, 16); break;
      default: IBP_CPR(16, 8, 4); break;
    }
#undef IBP_CPR
  } else if (n <= 1024)
    launch_compress_positional_t<1024>(table, n, n_rows, src, slots, flags, row_bits, st);
  else if (n <= 4096)
    launch_compress_positional_t<4096>(table, n, n_rows, src, slots, flags, row_bits, st);
  else if (n <= 8192)
    launch_compress_positional_t<8192>(table, n, n_rows, src, slots, flags, row_bits, st);
  else
    launch_compress_positional_t<IBP_MAX_COMPRESS_ROW_BYTES / 4>(table, n, n_rows, src, slots,
                                                                 flags, row_bits, st);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

static int decode_positional(const void* table, uint64_t n_rows, uint64_t row_bytes,
                             const void* slots, const uint64_t* flags, const int64_t* ids,
                             uint64_t n_out, void* dst, void* stream, bool gather) {
  if (!table) return IBP_ERR_INVALID_ARGUMENT;
  int rc = check_rows(n_rows, row_bytes);
  if (rc) return rc;
  if (n_out > UINT64_MAX / row_bytes) return IBP_ERR_INVALID_ARGUMENT;
  if (n_out == 0) return IBP_OK;
  if (n_rows == 0 || !slots || !flags || !dst || (gather && !ids)) return IBP_ERR_INVALID_ARGUMENT;
  if (!aligned(table, 16) || !aligned(slots, 4) || !aligned(dst, 4) || !aligned(flags, 8) ||
      (gather && !aligned(ids, 8)))
    return IBP_ERR_LAYOUT;
  rc = pending_hip_error();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  const uint32_t n = (uint32_t)(row_bytes / 4);
  const int vec = row_bytes % 16 == 0 && aligned(slots, 16) && aligned(dst, 16);
  if (vec && (n == 128 || n == 256 || n == 512 || n == 1024)) {
    // pipelined kernel, in launches of at most 2^30 rows (32-bit row indices)
    const uint64_t piece = 1ull << 30;
    for (uint64_t off = 0; off < n_out; off += piece) {
      const uint32_t cnt = (uint32_t)std::min<uint64_t>(piece, n_out - off);
      const uint32_t* sl = (const uint32_t*)slots;
      const unsigned long long* fl = (const unsigned long long*)flags;
      if (!gather) {  // rows off.. of the table; flags stay word aligned (piece % 64 == 0)
        sl += off * n;
        fl += off / 64;
      }
      const int64_t* id_p = gather ? ids + off : nullptr;
      uint32_t* out_p = (uint32_t*)dst + off * n;
      // workgroups of 4 waves (8 for 4 KiB rows, whose 32 KiB table is then
      // shared by more waves); per CU, measured: 6 for rows of 128 and 256
      // blocks (against 4, 5, 7, 8 and 12), 3 for 512 (against 2, 4, 5, 8),
      // 2 for 1024 (against 1, 3, 4): fewer workgroups stage the position
      // table fewer times
#define IBP_PP(G, NCH, WPB, PER_CU)                                                             \
  hipLaunchKernelGGL((decode_pos_pipe_kernel<G, NCH, WPB>), dim3(row_pipe_grid(cnt, WPB, PER_CU)), \
                     dim3(WPB * kWave), 0, st, (const PosEntry*)table, sl, fl, id_p,           \
                     gather ? n_rows : (uint64_t)cnt, cnt, out_p)
#define IBP_PP_N(G)                                         \
  switch (n) {                                              \
    case 128: IBP_PP(G, 2, 4, 6); break;                    \
    case 256: IBP_PP(G, 4, 4, 6); break;                    \
    case 512: IBP_PP(G, 8, 4, 3); break;                    \
    default: IBP_PP(G, 16, 8, 2); break;                    \
  }
      if (gather) { IBP_PP_N(true); } else { IBP_PP_N(false); }
#undef IBP_PP_N
#undef IBP_PP
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? IBP_OK : hip_fail(e);
  }
  const uint64_t wgs = (n_out + kWavesPerBlock - 1) / kWavesPerBlock;
  // with the table in LDS (48.5 KiB per workgroup): three workgroups per CU
  // are resident, and the table copy is paid once per workgroup
  const bool lds_table = n <= kSegBlocks;
  const uint32_t grid =
      (uint32_t)std::min<uint64_t>(wgs, workgroups_per_device(lds_table ? 3 : 8));
#define IBP_POS(G, TAB)                                                                    \
  hipLaunchKernelGGL((decode_positional_kernel<G, TAB>), dim3(grid), dim3(kBlockThreads), 0, \
                     st, (const PosEntry*)table, n, (const uint32_t*)slots,                 \
                     (const unsigned long long*)flags, G ? ids : nullptr, n_rows, n_out,   \
                     (uint32_t*)dst, vec)
  if (gather) {
    if (lds_table) IBP_POS(true, kSegBlocks); else IBP_POS(true, 0);
  } else {
    if (lds_table) IBP_POS(false, kSegBlocks); else IBP_POS(false, 0);
  }
#undef IBP_POS
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? IBP_OK : hip_fail(e);
}

int ibp_decompress_positional(const void* table, uint64_t n_rows, uint64_t row_bytes,
                              const void* slots, const uint64_t* flags, void* dst, void* stream) {
  return decode_positional(table, n_rows, row_bytes, slots, flags, nullptr, n_rows, dst, stream,
                           false);
}

int ibp_gather_decompress_positional(const void* table, uint64_t n_rows, uint64_t row_bytes,
                                     const void* slots, const uint64_t* flags,
                                     const int64_t* row_ids, uint64_t n_ids, void* dst,
                                     void* stream) {
  return decode_positional(table, n_rows, row_bytes, slots, flags, row_ids, n_ids, dst, stream,
                           true);
}

int ibp_host_device_pointer(const void* host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr) return IBP_ERR_INVALID_ARGUMENT;
  const int rc = pending_hip_error();
  if (rc) return rc;
  hipError_t e = hipHostGetDevicePointer(device_ptr, const_cast<void*>(host_ptr), 0);
  if (e == hipSuccess) return IBP_OK;
  (void)hipGetLastError();  // the status carries it; later HIP calls start clean
  return hip_fail(e);
}

}  // extern "C"
