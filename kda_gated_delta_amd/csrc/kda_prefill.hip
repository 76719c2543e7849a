// Chunkwise varlen prefill of the KDA gated delta rule.
//
// The recurrence ("Linear attention" tutorial, section "KDA：逐通道的遗忘门")
//   S_t = (I - b_t k_t^T k_t) Diag(exp g_t) S_{t-1} + b_t k_t^T v_t,  o_t = scale q_t S_t
// is evaluated a chunk of C tokens at a time (section "两种计算形态": the C
// rank-1 updates of a chunk merge through the WY/UT representation and one
// C x C triangular solve; only the state crosses chunk boundaries).
//
// Unrolling one chunk (G = inclusive chunk-local cumulative sum of g, S0 the
// state entering the chunk, B = diag(beta)):
//   A[t,j]  = sum_c k_t[c] k_j[c] exp(G_t[c] - G_j[c])   (j <  t)
//   Aq[t,j] = sum_c q_t[c] k_j[c] exp(G_t[c] - G_j[c])   (j <= t)
//   X = (I + B A)^-1 (unit lower triangular),  M = X B
//   W = M (K * e^G),  U = M V,  D = U - W S0
//   O = scale [ (Q * e^G) S0 + Aq D ]
//   S_C = Diag(e^{G_C}) S0 + (K * e^{G_C - G})^T D
// Every exponent used is <= 0 (never overflows): inside A and Aq only
// G_t - G_j with t >= j appears; off-diagonal 16 x 16 blocks factor through
// the first row r of the row block, exp(G_t - G_r) exp(G_r - G_j), both <= 1.
//
// Three kernels:
//   plan   - one workgroup: chunk table of the packed batch from cu_seqlens
//            (clamped into [0, T], so a malformed array cannot push an
//            access out of bounds);
//   intra  - one workgroup per (chunk, head), fully parallel: everything of a
//            chunk that does not depend on the carried state (G, A, Aq, the
//            triangular inverse, W, U, Q*e^G, K*e^{G_C-G}), written to the
//            workspace already in MFMA fragment order;
//   state  - one workgroup per (sequence, head, V tile), serial over the
//            chunks of its sequence: D, O and the state update, with the
//            state tile resident in MFMA accumulators.
// Contractions use v_mfma_f32_16x16x32_bf16 with every fp32 operand split
// into bf16 hi + lo parts (three products, fp32 accumulation): relative error
// about 2^-16 per product, enough for fp32 inputs; the cumulative sums, the
// exponentials and the triangular inverse are fp32 on the vector ALUs.

#include "kda_common.h"
#include "kda_gate_math.h"
#include "kda_internal.h"

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NTHREADS = 256;  // four waves per workgroup

// -------------------------------------------------------------- fragments
//
// v_mfma_f32_16x16x32_bf16, lane l (0..63), g = l / 16, r = l % 16:
//   A operand (16 x 32, row-major): A[r][8g + j], j = 0..7
//   B operand (32 x 16):            B[8g + j][r]
//   accumulator (16 x 16):          C[4g + i][r], i = 0..3

struct Frag {
  bf16x8 hi, lo;
};

//
// hi = bf16(x) (round to nearest even, two values per v_cvt_pk_bf16_f32) and
// lo = bf16(x - hi).  x - hi is exact in fp32; it is taken as one v_dot2 of
// the packed hi pair with (-1, 0) or (0, -1), plus x, which saves the
// bf16 -> fp32 unpack.  The pair's other element enters as 0 * h: zero for
// every finite h (an infinite h, from an overflowed x, makes both lo NaN).
// The two multipliers are kept in scalar registers (materialised by asm):
// the compiler would otherwise encode (-1, 0) as the inline constant -1.0,
// which the hardware reads as the fp32 value, i.e. as the pair (0, -1).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ Frag split8(const float (&x)[8]) {
  unsigned m0, m1;
  asm("s_mov_b32 %0, 0x0000bf80" : "=s"(m0));  // (-1, 0)
  asm("s_mov_b32 %0, 0xbf800000" : "=s"(m1));  // (0, -1)
  Frag f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bf16x2 h = {(bf16)x[2 * p], (bf16)x[2 * p + 1]};
    const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m0), x[2 * p], false);
    const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m1), x[2 * p + 1], false);
    f.hi[2 * p] = h[0];
    f.hi[2 * p + 1] = h[1];
    f.lo[2 * p] = (bf16)l0;
    f.lo[2 * p + 1] = (bf16)l1;
  }
  return f;
}

// acc += a * b with a, b given as hi + lo (the lo * lo term is dropped).
__device__ __forceinline__ f32x4 mma3(f32x4 acc, const Frag& a, const Frag& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
  return acc;
}

// A fragment tile stored in the workspace: 64 lanes x 16 B of hi parts, then
// 64 lanes x 16 B of lo parts (each half one coalesced 1 KB wave access).
constexpr int FRAG_BYTES = 2048;

__device__ __forceinline__ void store_frag(char* tile, const Frag& f) {
  const int l = threadIdx.x & 63;
  *reinterpret_cast<bf16x8*>(tile + l * 16) = f.hi;
  *reinterpret_cast<bf16x8*>(tile + 1024 + l * 16) = f.lo;
}

__device__ __forceinline__ Frag load_frag(const char* tile) {
  const int l = threadIdx.x & 63;
  Frag f;
  f.hi = *reinterpret_cast<const bf16x8*>(tile + l * 16);
  f.lo = *reinterpret_cast<const bf16x8*>(tile + 1024 + l * 16);
  return f;
}

// Buffer-resource loads (buffer_rsrc in kda_common.h): the base and every
// tile offset stay in scalar registers, the only per-lane address is the
// lane's 16-byte slot.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A fragment tile at byte `tile` of the resource (hi plane, then lo plane).
__device__ __forceinline__ Frag buffer_frag(__amdgpu_buffer_rsrc_t r, uint32_t lane16,
                                            uint32_t tile) {
  Frag f;
  f.hi = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, lane16, tile, 0));
  f.lo = __builtin_bit_cast(bf16x8,
                            __builtin_amdgcn_raw_buffer_load_b128(r, lane16, tile + 1024, 0));
  return f;
}

__device__ __forceinline__ f32x4 buffer_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Scheduling hint for the block it sits in: spread `loads` vector-memory
// reads evenly over the first `mfmas` MFMAs, so that a burst of loads does
// not stall the wave on a full memory queue.
template <int MFMAS, int LOADS>
__device__ __forceinline__ void interleave_loads() {
  constexpr int PER = MFMAS / LOADS > 0 ? MFMAS / LOADS : 1;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read
  }
}

// Eight consecutive values (16-byte aligned) from LDS as fp32.
__device__ __forceinline__ void lds8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void lds8(const bf16* p, float (&x)[8]) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)a[j];
}

// ------------------------------------------------------- workspace layout

struct ChunkEntry {
  int seq, start, len, pad;
};

template <int D, int C>
struct Geom {
  static constexpr int NB = C / 16;          // 16-row blocks of a chunk
  static constexpr int KTC = (C + 31) / 32;  // 32-wide k steps over tokens
  static constexpr int KTD = (D + 31) / 32;  // 32-wide k steps over channels
  static constexpr int MTD = D / 16;         // 16-row tiles over channels
  // per (chunk, head) record, in bytes
  static constexpr size_t W_OFF = 0;                                  // [NB][KTD] A frags
  static constexpr size_t Q_OFF = W_OFF + (size_t)NB * KTD * FRAG_BYTES;  // [NB][KTD]
  static constexpr size_t KT_OFF = Q_OFF + (size_t)NB * KTD * FRAG_BYTES;  // [MTD][KTC]
  static constexpr size_t AQ_OFF = KT_OFF + (size_t)MTD * KTC * FRAG_BYTES;  // [NB][KTC]
  static constexpr size_t U_OFF = AQ_OFF + (size_t)NB * KTC * FRAG_BYTES;  // [NB][MTD] acc tiles
  static constexpr size_t GC_OFF = U_OFF + (size_t)NB * MTD * 64 * 16;    // [D] fp32
  static constexpr size_t REC = ((GC_OFF + D * 4) + 255) / 256 * 256;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Per-sequence plan entry: the clamped token range lo .. hi-1, the first
// chunk of the sequence in the chunk table, the first snapshot row, and,
// when the sequence is cut into segments, its first start-state slot and
// first map slot.
struct SeqInfo {
  int lo, hi, chunk_first, snap_base, start_slot, map_slot, pad0, pad1;
};

// A work unit of the state pass: the chunk-table entries c_begin .. c_end-1,
// chunks r_begin, r_begin + 1, .. of sequence `seq`, in one of three roles.
//  - a segment of the chain (the whole sequence when it is not cut): from
//    h0 (or zeros) or, with UNIT_FROM_START, from start slot in_slot; it
//    writes ht when it ends the sequence (UNIT_WRITE_HT), else its final
//    state into start slot out_slot (UNIT_WRITE_NEXT), the next segment's
//    start;
//  - the map of a middle segment: the affine map S -> M S + B of its chunks,
//    computed as the state pass over the K + V columns of [M | B] from
//    [I | 0] with no read-out, into map slot out_slot.
// A unit without flags (a wave the sequence does not reach) does nothing.
// A chunk is the affine map S -> (Diag(e^{G_C}) - (K e^{G_C-G})^T W) S +
// (K e^{G_C-G})^T U, and maps compose because the decay is diagonal
// ("ReplaySSM" analysis, section 2.1): a long sequence's serial chain of
// chunks can be cut into segments whose maps are built side by side, chained
// by a short scan, and re-run from their true starts.  Cut into waves of
// consecutive segments instead, the chain stays whole (the state is handed
// on exactly through the start slots) and wave p's state pass can run while
// the intra-chunk work of wave p + 1 is still being done.
enum { UNIT_WRITE_HT = 1, UNIT_WRITE_NEXT = 2, UNIT_FROM_START = 4 };
struct Unit {
  int seq, c_begin, c_end, flags, in_slot, out_slot, r_begin, pad;
};

// How the state pass is cut (decided on the host from T, N, H, D, C alone:
// the host never reads the sequence lengths, so every choice assumes the
// worst case for the chain, one sequence of all T tokens).
//  - maps: when the batch's (sequence, head) chains leave most of a 256-CU
//    chip idle (one state workgroup per CU), middle segments build their
//    chunk maps side by side.  The segment count P (smooth values; 16 even
//    segments of 64 chunks beat 17 of 61 by 15% on one 65536-token
//    sequence) minimises the chunk steps on the critical path: the first
//    launch runs the first segments and the maps, the maps beyond the chip's
//    width in further rounds (a full step per round: a map workgroup carries
//    as many columns as a state one, without the read-out but with twice the
//    workgroups); the second launch re-runs the P - 1 later segments; the
//    scan adds about 0.6 of a step per segment.  (Fitted to the 65536-token
//    sequence at H = 4: 32, 16 and 8 segments measured 459, 421 and 545 us.)
//    Taken only when that beats the whole chain by a quarter.
//  - waves: otherwise, when the chains still leave CUs free (so that the
//    intra-chunk kernel has room beside the state pass) and a chain can
//    reach 128 chunks, the chain is cut into about 8 waves of at least 16
//    chunks, handed on exactly, and the intra-chunk work of each wave
//    overlaps the state pass of the previous.  (On the packed 7680-token
//    batch, whose 512 chains fill the chip, waves cost 30% more than they
//    save; on one 65536-token sequence they save 13%.)
constexpr int STATE_CUS = 256;
struct StateCut {
  int seg_len;   // chunks per segment (0: the chain is never cut)
  bool maps;     // segments chained by maps (else: waves)
  int n_waves;   // waves of the pipelined schedule (1 without)
};

StateCut state_cut(int64_t T, int N, int H, int D, int C) {
  StateCut cut{0, false, 1};
  const int VT = D >= 32 ? 32 : D;
  const int64_t NV = D / VT, NM = 2 * NV;
  const int64_t nch = (T + C - 1) / C;
  if ((int64_t)N * H * NV < STATE_CUS && nch >= 128) {
    auto rounds = [](int64_t units) { return (units + STATE_CUS - 1) / STATE_CUS; };
    double best = 0.75 * (double)nch;
    static const int64_t kSegments[] = {3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
    for (const int64_t P : kSegments) {
      const int64_t len = (nch + P - 1) / P;
      if (len < 32) break;
      const int64_t first = (int64_t)N * H * NV, maps = (P - 2) * H * NM;
      const int64_t spill = first + maps > STATE_CUS ? first + maps - STATE_CUS : 0;
      const double a = 1.0 + (double)rounds(spill);
      const double c = (double)rounds((P - 1) * H * NV);
      const double cost = (a + c) * (double)len + 0.6 * (double)(P - 2);
      if (cost < best) {
        best = cost;
        cut.seg_len = (int)len;
        cut.maps = true;
      }
    }
  }
  if (!cut.maps && (int64_t)N * H * NV <= STATE_CUS && nch >= 128) {
    cut.seg_len = (int)std::max<int64_t>(16, (nch + 7) / 8);
    cut.n_waves = (int)((nch + cut.seg_len - 1) / cut.seg_len);
  }
  return cut;
}

// Header of the workspace: chunk table [NCB] (wave-major with waves,
// sequence-major otherwise), per-sequence entries [N], the state pass's
// units (first segments [N] in the order the pass takes them, maps and later
// segments, at most NSEG each; with waves, [waves, N] units instead), the
// unit counts and the waves' chunk-table offsets, then the per-chunk
// records, and with a cut chain the start states [NSEG, H, D, D] and maps
// [NSEG, H, D, 2 D] (fp32; each map in 4-column tiles, see state_unit).
struct WsLayout {
  size_t table_off, seq_off, unit_a_off, unit_m_off, unit_c_off, unit_w_off, count_off,
      wave_off, rec_off, start_off, map_off, total;
  int64_t ncb, nseg;
  StateCut cut;
};

WsLayout ws_layout(int64_t T, int N, int H, int D, int C, size_t rec) {
  WsLayout w;
  w.ncb = (T + C - 1) / C + N;
  w.cut = state_cut(T, N, H, D, C);
  w.nseg = w.cut.seg_len > 0 ? w.ncb / w.cut.seg_len + N : 0;
  const int64_t nmaps = w.cut.maps ? w.nseg : 0;
  const int64_t nwunits = w.cut.n_waves > 1 ? (int64_t)w.cut.n_waves * N : 0;
  w.table_off = 0;
  w.seq_off = round256((size_t)w.ncb * sizeof(ChunkEntry));
  w.unit_a_off = w.seq_off + round256((size_t)N * sizeof(SeqInfo));
  w.unit_m_off = w.unit_a_off + round256((size_t)N * sizeof(Unit));
  w.unit_c_off = w.unit_m_off + round256((size_t)nmaps * sizeof(Unit));
  w.unit_w_off = w.unit_c_off + round256((size_t)(w.cut.maps ? w.nseg : 0) * sizeof(Unit));
  w.count_off = w.unit_w_off + round256((size_t)nwunits * sizeof(Unit));
  w.wave_off = w.count_off + 256;
  w.rec_off = w.wave_off + round256((size_t)(w.cut.n_waves + 1) * sizeof(int));
  w.start_off = w.rec_off + (size_t)w.ncb * H * rec;
  w.map_off = w.start_off + (size_t)w.nseg * H * D * D * 4;
  w.total = w.map_off + (size_t)nmaps * H * D * 2 * D * 4;
  return w;
}

size_t rec_bytes(int D, int C) {
#define KDA_REC(d, c) \
  if (D == d && C == c) return Geom<d, c>::REC;
  KDA_REC(16, 16) KDA_REC(16, 32) KDA_REC(16, 64)
  KDA_REC(32, 16) KDA_REC(32, 32) KDA_REC(32, 64)
  KDA_REC(64, 16) KDA_REC(64, 32) KDA_REC(64, 64)
  KDA_REC(128, 16) KDA_REC(128, 32) KDA_REC(128, 64)
#undef KDA_REC
  return 0;
}

// ------------------------------------------------------------------- plan

// Inclusive scan over the NTHREADS threads of a workgroup (Hillis-Steele in
// LDS); `op` is max or +.  Every thread must call it.
template <typename Op>
__device__ __forceinline__ int block_scan(int x, int* scratch, Op op) {
  const int t = threadIdx.x;
  scratch[t] = x;
  __syncthreads();
  for (int s = 1; s < NTHREADS; s <<= 1) {
    const int y = t >= s ? scratch[t - s] : x;
    __syncthreads();
    if (t >= s) x = op(x, y);
    scratch[t] = x;
    __syncthreads();
  }
  return x;
}

// Chunk table of the packed batch.  Sequence bounds are made disjoint and
// monotone whatever cu_seqlens holds: with c'_m = min(max(cu[m], 0), T) and
// p_n = max(c'_0 .. c'_n), sequence n owns tokens p_n .. p_{n+1}-1.  For a
// valid cu_seqlens (cu[0] = 0 <= cu[1] <= .. <= cu[N] = T) that is exactly
// cu[n] .. cu[n+1]-1; for any other array the ranges still partition a part
// of [0, T), so the chunks never outnumber the workspace's ceil(T/C) + N.
// Table entries past the last chunk get len = 0.  With snapshots, sequence n
// owns the rows from seqs[n].snap_base on, floor((hi - lo) / snap_interval)
// of them.  The state pass's units follow the cut (see StateCut): with
// segments of seg_len chunks, a sequence of nch chunks has ceil(nch /
// seg_len) of them (one when nch <= seg_len) and one start slot per segment
// after its first.  Without waves the table is sequence-major (sequence n
// owns entries chunk_first .. + nch - 1); with n_waves > 1 it is wave-major:
// wave p holds segment p of every sequence that has one, sequence after
// sequence, from entry wave_off[p] on.
__global__ __launch_bounds__(NTHREADS) void plan_kernel(
    const int32_t* __restrict__ cu, int N, int64_t T, int C, int64_t ncb, int snap_interval,
    int seg_len, int maps, int n_waves, ChunkEntry* __restrict__ table,
    SeqInfo* __restrict__ seqs, Unit* __restrict__ units_a, Unit* __restrict__ units_m,
    Unit* __restrict__ units_c, Unit* __restrict__ units_w, int* __restrict__ counts,
    int* __restrict__ wave_off) {
  __shared__ int scratch[NTHREADS];
  __shared__ int carry_max, carry_chunks, carry_snaps, carry_starts, carry_maps, carry_wave;
  __shared__ int bcount[33], bbase[33];
  const int t = threadIdx.x;
  const bool waves = n_waves > 1;
  auto clampT = [&](int64_t x) { return (int)(x < 0 ? 0 : (x > T ? T : x)); };
  auto bucket_of = [](int nch) { return nch <= 0 ? 0 : 32 - __clz(nch); };
  auto imax = [](int a, int b) { return a > b ? a : b; };
  auto iadd = [](int a, int b) { return a + b; };
  auto nseg_of = [&](int nch) {
    return seg_len > 0 && nch > seg_len ? (nch + seg_len - 1) / seg_len : 1;
  };
  auto unit = [](int seq, int c_begin, int c_end, int flags, int in_slot, int out_slot,
                 int r_begin) {
    Unit u;
    u.seq = seq;
    u.c_begin = c_begin;
    u.c_end = c_end;
    u.flags = flags;
    u.in_slot = in_slot;
    u.out_slot = out_slot;
    u.r_begin = r_begin;
    u.pad = 0;
    return u;
  };
  if (t == 0) {
    carry_max = clampT(cu[0]);
    carry_chunks = 0;
    carry_snaps = 0;
    carry_starts = 0;
    carry_maps = 0;
  }
  if (t < 33) bcount[t] = 0;
  __syncthreads();
  // ---- per sequence: bounds, chunks, snapshot rows, start and map slots
  for (int base = 0; base < N; base += NTHREADS) {
    const int n = base + t;
    const int cm = carry_max, cc = carry_chunks, cs = carry_snaps;
    const int cst = carry_starts, cmp = carry_maps;
    // hi of sequence n = p_{n+1}; lo = hi of sequence n-1 (p_n)
    const int hi = imax(cm, block_scan(n < N ? clampT(cu[n + 1]) : 0, scratch, imax));
    const int lo = t == 0 ? cm : imax(cm, scratch[t - 1]);
    const int len = n < N ? hi - lo : 0;
    const int nch = (len + C - 1) / C;
    const int nsn = snap_interval > 0 ? len / snap_interval : 0;
    __syncthreads();
    const int first = cc + block_scan(nch, scratch, iadd) - nch;
    __syncthreads();
    const int sfirst = cs + block_scan(nsn, scratch, iadd) - nsn;
    const int nseg = n < N ? nseg_of(nch) : 1;
    __syncthreads();
    const int stfirst = cst + block_scan(nseg - 1, scratch, iadd) - (nseg - 1);
    const int nmap = maps && nseg > 2 ? nseg - 2 : 0;
    __syncthreads();
    const int mfirst = cmp + block_scan(nmap, scratch, iadd) - nmap;
    if (n < N) {
      SeqInfo e;
      e.lo = lo;
      e.hi = hi;
      e.chunk_first = first;
      e.snap_base = sfirst;
      e.start_slot = stfirst;
      e.map_slot = mfirst;
      e.pad0 = e.pad1 = 0;
      seqs[n] = e;
      atomicAdd(&bcount[bucket_of(nch)], 1);
      if (maps) {
        // the maps of the middle segments and the re-runs of the later ones
        for (int p = 1; p < nseg; ++p) {
          const int b0 = first + p * seg_len, b1 = min(first + (p + 1) * seg_len, first + nch);
          units_c[stfirst + p - 1] = unit(n, b0, b1,
                                          UNIT_FROM_START | (p == nseg - 1 ? UNIT_WRITE_HT : 0),
                                          stfirst + p - 1, -1, p * seg_len);
          if (p < nseg - 1)
            units_m[mfirst + p - 1] = unit(n, b0, b1, 0, -1, mfirst + p - 1, p * seg_len);
        }
      }
    }
    __syncthreads();
    if (t == NTHREADS - 1) {
      carry_max = hi > cm ? hi : cm;
      carry_chunks = first + nch;
      carry_snaps = sfirst + nsn;
      carry_starts = stfirst + nseg - 1;
      carry_maps = mfirst + nmap;
    }
    __syncthreads();
  }
  if (t == 0) {
    counts[0] = N;             // first segments (every sequence)
    counts[1] = carry_maps;    // middle-segment maps
    counts[2] = carry_starts;  // later segments
  }
  const int total = carry_chunks;  // <= ncb (see above)
  __threadfence_block();
  __syncthreads();
  // ---- waves: segment p of every sequence, in wave-major table order
  if (waves) {
    if (t == 0) carry_wave = 0;
    __syncthreads();
    for (int p = 0; p < n_waves; ++p) {
      if (t == 0) wave_off[p] = carry_wave;
      for (int base = 0; base < N; base += NTHREADS) {
        const int n = base + t;
        const int cw = carry_wave;
        SeqInfo e{};
        int cnt = 0;
        if (n < N) {
          e = seqs[n];
          const int nch = (e.hi - e.lo + C - 1) / C;
          cnt = min(max(nch - p * seg_len, 0), seg_len);
        }
        __syncthreads();
        const int off = cw + block_scan(cnt, scratch, iadd) - cnt;
        if (n < N) {
          const int nch = (e.hi - e.lo + C - 1) / C;
          const int nseg = nseg_of(nch);
          int flags = 0;
          if (p < nseg)
            flags = (p > 0 ? UNIT_FROM_START : 0) |
                    (p < nseg - 1 ? UNIT_WRITE_NEXT : UNIT_WRITE_HT);
          units_w[(size_t)p * N + n] =
              unit(n, off, off + cnt, flags, e.start_slot + p - 1, e.start_slot + p, p * seg_len);
        }
        __syncthreads();
        if (t == NTHREADS - 1) carry_wave = off + cnt;
        __syncthreads();
      }
    }
    if (t == 0) wave_off[n_waves] = carry_wave;
    __threadfence_block();
    __syncthreads();
  } else if (t == 0) {
    wave_off[0] = 0;
    wave_off[1] = total;
  }
  // Longest sequences first: units_a lists the sequences' first segments by
  // descending power-of-two bucket of their chunk count, so the state pass
  // starts the longest serial chains first.
  if (t == 0) {
    int acc = 0;
    for (int b = 32; b >= 0; --b) {
      bbase[b] = acc;
      acc += bcount[b];
    }
  }
  __syncthreads();
  for (int n = t; n < N; n += NTHREADS) {
    const SeqInfo e = seqs[n];
    const int nch = (e.hi - e.lo + C - 1) / C;
    const int pos = atomicAdd(&bbase[bucket_of(nch)], 1);
    // the first (or only) segment of sequence n, sequence-major
    const int nseg = nseg_of(nch);
    units_a[pos] = unit(n, e.chunk_first, e.chunk_first + (nseg > 1 ? seg_len : nch),
                        nseg > 1 ? UNIT_WRITE_NEXT : UNIT_WRITE_HT, -1, e.start_slot, 0);
  }
  // table entry i: sequence-major, entry i belongs to the last sequence
  // whose first chunk is <= i; wave-major, to the last unit of its wave that
  // begins at or before i (binary searches over monotone offsets: empty
  // sequences or units share their successor's offset and lose them)
  for (int64_t i = t; i < ncb; i += NTHREADS) {
    ChunkEntry e;
    e.seq = 0;
    e.start = 0;
    e.len = 0;
    e.pad = 0;
    if (i < total) {
      int n, r;
      if (waves) {
        int a = 0, b = n_waves - 1;  // last wave p with wave_off[p] <= i
        while (a < b) {
          const int m = (a + b + 1) >> 1;
          if (wave_off[m] <= i) a = m; else b = m - 1;
        }
        const Unit* U = units_w + (size_t)a * N;
        int c = 0, d = N - 1;  // last n with U[n].c_begin <= i
        while (c < d) {
          const int m = (c + d + 1) >> 1;
          if (U[m].c_begin <= i) c = m; else d = m - 1;
        }
        n = c;
        r = U[c].r_begin + ((int)i - U[c].c_begin);
      } else {
        int a = 0, b = N - 1;  // last m with chunk_first <= i
        while (a < b) {
          const int m = (a + b + 1) >> 1;
          if (seqs[m].chunk_first <= i) a = m; else b = m - 1;
        }
        n = a;
        r = (int)i - seqs[a].chunk_first;
      }
      const SeqInfo s = seqs[n];
      e.seq = n;
      e.start = s.lo + r * C;
      e.len = (s.hi - e.start < C) ? s.hi - e.start : C;
    }
    table[i] = e;
  }
}

// ------------------------------------------------------------------ intra

// Swizzled LDS layouts (no padding).  A row of N elements is cut into groups
// of GR elements; group i of row r is stored at group position i ^ (r mod
// N/GR).  Lanes that read the same columns of different rows then hit
// different banks, and a group stays contiguous.
template <int N, int GR>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int NG = N / GR;
  static_assert((NG & (NG - 1)) == 0 && (GR & (GR - 1)) == 0, "powers of two");
  return r * N + ((((unsigned)c / GR) ^ (unsigned)r) & (NG - 1)) * GR + ((unsigned)c % GR);
}

constexpr int NT_INTRA = 512;  // eight waves: two per SIMD

template <typename IO, int D, int C>
struct IntraSmem {
  static constexpr int NB = C / 16, KTC = (C + 31) / 32;
  // row groups of the cumulative-sum staging (step 1): NT_INTRA / (D / 4)
  // groups of RPT rows, NU of which hold rows
  static constexpr int NGR = NT_INTRA / (D / 4), RPT = (C + NGR - 1) / NGR;
  static constexpr int NU = (C + RPT - 1) / RPT;
  static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
  // sG [C][D] fp32: G (groups of 8), then K e^G and V (plain)
  static constexpr size_t G_BYTES = (size_t)C * D * 4;
  // sK [C][D] io (groups of 8): k; then the block-inverse scratch; then the
  // split fragments of M = X diag(beta)
  static constexpr size_t K_BYTES = cmax(cmax((size_t)C * D * sizeof(IO),
                                              (size_t)NB * KTC * FRAG_BYTES),
                                         (size_t)6 * 256 * 4);
  // sQ [C][D] io (groups of 8): q; then beta
  static constexpr size_t Q_BYTES = cmax((size_t)C * D * sizeof(IO), (size_t)C * 4);
  // sAA [C][C] fp32 (plain): first the NU row-group totals of step 1 and,
  // past them, the inverse norms of q and k rows; then A transposed in the
  // strict upper triangle and Aq in the lower one, Aq's triangle then reused
  // for X; finally the 32-row staging of W ([32][D] fp32, groups of 8)
  static constexpr size_t AA_BYTES =
      cmax(cmax((size_t)C * C * 4, (size_t)32 * D * 4), (size_t)(NU * D + 2 * C) * 4);
  static constexpr size_t TOTAL = G_BYTES + K_BYTES + Q_BYTES + AA_BYTES;
};

// Cache policy of the intra kernel's streams (inputs read once, records
// written once and read by the next kernel): the non-temporal hint.
constexpr int NT_HINT = 2;

// Off-diagonal work of A and Aq: wave NB + idx takes row block I and the
// column blocks J0 .. J0 + nJ - 1 (at most two, sharing the row operand);
// row blocks are dealt from the last one.
template <int NB>
__device__ __forceinline__ void offdiag_group(int idx, int& I, int& J0, int& nJ) {
  int k = 0;
  I = 0;
  J0 = 0;
  nJ = 0;
#pragma unroll
  for (int i = NB - 1; i >= 1; --i)
#pragma unroll
    for (int j = 0; j < i; j += 2) {
      if (k == idx) {
        I = i;
        J0 = j;
        nJ = (i - j) < 2 ? (i - j) : 2;
      }
      ++k;
    }
}

// The intra pass keeps G log2(e) in LDS: e^{G_a - G_b} is then one base-2
// exponential (v_exp_f32) of the difference of two stored values.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of squares of one 16-byte group of io elements (raw bits).
template <typename IO>
__device__ __forceinline__ float sumsq16(const uint4 x) {
  float s = 0.f;
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(IO) == 2) {  // bf16 pairs: element 2i in the low half of word i
      const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
      s = fmaf(lo, lo, fmaf(hi, hi, s));
    } else {
      const float f = __uint_as_float(w[i]);
      s = fmaf(f, f, s);
    }
  }
  return s;
}

// One step of a transposing reduction over a 16-lane row: the lane's first
// 2 H sums are halved into H, keeping the upper half when `upper` (the index
// bit of this step) is set and adding the partner lane's copy of the same
// half, fetched by the DPP control CTRL.
template <int H, int CTRL>
__device__ __forceinline__ void butterfly_step(float (&v)[16], int upper) {
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const float send = upper ? v[j] : v[H + j];
    const float keep = upper ? v[H + j] : v[j];
    v[j] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xf, 0xf, false));
  }
}

// LDS use (bf16 io, C = 64, D = 128: 80 KB, two workgroups per CU): see
// IntraSmem.  Every input is staged once; the work units read their rows
// from LDS into registers and take reference rows by lane broadcast.
// GATE: the gate form compiled into the instance: 0 = g and beta are given,
// 1 = softplus gate, 2 = safe gate applied to the raw inputs (one form per
// instance, so that no instance carries another's code; the three show up as
// separate kernels in a profile).
template <typename IO, int D, int C, int GATE>
__global__ __launch_bounds__(NT_INTRA, 4) void intra_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, int H, float scale,
    const ChunkEntry* __restrict__ table, char* __restrict__ recs,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, float lower_bound,
    int HK, int per_head_gate, int qk_l2norm, int ncb, const int* __restrict__ wave_off,
    int wave) {
  typedef Geom<D, C> Gm;
  typedef IntraSmem<IO, D, C> Sm;
  constexpr int NT = NT_INTRA, NW = NT / 64;
  constexpr int NB = Gm::NB, KTC = Gm::KTC, KTD = Gm::KTD, MTD = Gm::MTD;
  constexpr int IOV = 16 / (int)sizeof(IO);  // io elements per 16 bytes
  __shared__ __align__(16) char smem[Sm::TOTAL];
  float* sG = reinterpret_cast<float*>(smem);
  IO* sK = reinterpret_cast<IO*>(smem + Sm::G_BYTES);
  float* sY = reinterpret_cast<float*>(smem + Sm::G_BYTES);     // over k (solve)
  bf16x8* sMf = reinterpret_cast<bf16x8*>(smem + Sm::G_BYTES);  // over k (W, U)
  IO* sQ = reinterpret_cast<IO*>(smem + Sm::G_BYTES + Sm::K_BYTES);
  float* sB = reinterpret_cast<float*>(smem + Sm::G_BYTES + Sm::K_BYTES);  // over q
  float* sAA = reinterpret_cast<float*>(smem + Sm::G_BYTES + Sm::K_BYTES + Sm::Q_BYTES);
  float* sW = sAA;  // W staging, over A / Aq / X

  // layouts
  auto iG = [](int t, int c) { return swz<D, 8>(t, c); };    // sG, sK, sQ
  auto iA = [](int r, int c) { return r * C + c; };          // sAA (plain)
  auto iP = [](int t, int c) { return t * D + c; };          // sG from step 5 (plain)
  auto iW = [](int r, int c) { return swz<D, 8>(r, c); };    // sW

  // the launch covers table entries wave_off[wave] .. wave_off[wave + 1] - 1
  // (every entry without waves); blocks past them return
  const int chunk = wave_off[wave] + (int)(blockIdx.x / H), h = blockIdx.x % H;
  if (chunk >= wave_off[wave + 1]) return;
  const ChunkEntry ce = table[chunk];
  if (ce.len <= 0) return;
  const int L = ce.len;
  // records are head-major, so that one head's chain of chunks is contiguous
  char* rec = recs + ((size_t)h * ncb + chunk) * Gm::REC;
  // Record stores go through one buffer resource per tile: the lane's byte
  // offset is their only per-lane operand and stays in one register for the
  // whole kernel, so no register an outstanding store addresses is ever
  // rewritten (which would make the wave wait for the store).  The scalar
  // offset operand stays the constant 0: with a register there, the compiler
  // lets the next instruction rewrite the store's data registers, and on this
  // chip that corrupts the stored data.
  const int tid = threadIdx.x, l = tid & 63, lg = l >> 4, lr = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lane16 = (uint32_t)l * 16;
  auto put_frag = [&](uint32_t off, const Frag& f) {
    const auto r = buffer_rsrc(rec + off, FRAG_BYTES);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f.hi), r, lane16, 0, NT_HINT);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f.lo), r, lane16 + 1024, 0, NT_HINT);
  };

  // Rows t = 0 .. L-1 of this chunk and head of a [T, H, width] tensor as a
  // buffer resource: element (t, c) sits at byte (t H width + c) esz, and
  // rows at or past L fall outside the range and read as zero.  Every load
  // below is unconditional, so a thread issues all of them back to back.
  auto rows = [&](const void* base, int width, int esz) {
    return buffer_rsrc(static_cast<const char*>(base) + ((size_t)ce.start * H + h) * width * esz,
                       (uint32_t)L * (uint32_t)(H * width * esz));
  };
  // q and k have HK heads: value head h reads head h / (H / HK) (grouped
  // value heads); rows of [T, HK, D]
  const int hk = h / (H / HK);
  auto qk_rows = [&](const void* base) {
    constexpr int esz = (int)sizeof(IO);
    return buffer_rsrc(static_cast<const char*>(base) + ((size_t)ce.start * HK + hk) * D * esz,
                       (uint32_t)L * (uint32_t)(HK * D * esz));
  };
  constexpr int gate_mode = GATE;
  // gate_mode 0: g and beta are given.  1 (softplus gate) and 2 (safe gate):
  // g and beta hold the raw inputs a and b, activated here with the gate
  // kernel's own functions (the same values it would have written); beta is
  // activated in step 5, where it is first stored.
  const float rate = gate_mode != 0 ? exp_split(A_log[h]) : 0.f;
  const float braw = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(rows(beta, 1, 4), (uint32_t)(tid * H * 4), 0, 0));

  // In-kernel L2 norm of q and k (option): 1 / sqrt(|row|^2 + 1e-6) of every
  // q and k row of the chunk, lane t of each wave holding row t's.  A row
  // enters every product linearly, so these factors scale the products'
  // results (A, Aq, the in-sub-block sums) and the state pass's operands
  // (scale Q e^G, K e^{G_C-G}, K e^G and through it W); q and k stay as given.
  // rq_of / rk_of must run with every lane of the wave active.
  float rq_all = 1.f, rk_all = 1.f;
  auto rq_of = [&](int t) { return __shfl(rq_all, t, 64); };
  auto rk_of = [&](int t) { return __shfl(rk_all, t, 64); };

  // ---- 1. stage g, k, q (rows t >= L are zero) with the chunk-local
  // inclusive cumulative sum of g folded in.  A thread holds RPT consecutive
  // rows of one four-channel group of g and scans them in registers; the
  // totals of the NU row groups pass through sAA (free until step 3), and
  // each thread adds those of the groups before its own.  sG keeps G log2(e),
  // so that every exponential below is a single base-2 exponential of a
  // difference.  All loads of a thread are issued before any LDS access.
  {
    constexpr int GQ = D / 4;                    // four-channel groups per row
    constexpr int NGR = NT / GQ;                 // row groups
    constexpr int RPT = (C + NGR - 1) / NGR;     // rows per thread
    constexpr int NU = (C + RPT - 1) / RPT;      // row groups that hold rows
    constexpr int K16 = (C * (D / IOV) + NT - 1) / NT;  // 16-byte groups of k, q
    static_assert(NU == Sm::NU && (NU * D + 2 * C) * 4 <= (int)Sm::AA_BYTES,
                  "group totals and row norms fit in sAA");
    const int cq = tid % GQ, grp = tid / GQ, c4 = 4 * cq;
    // A per-head gate (Gated DeltaNet: g [T, H], dt_bias [H]) is one value
    // per (token, head) that every channel shares.  It is read by the same
    // 16-byte loads, of the aligned group of four heads that holds h (H is a
    // multiple of 4), and the head's word is broadcast: no branch separates
    // the loads, so none of them waits for another.
    const int hsub = per_head_gate ? (h & 3) : 0;
    const auto rG = per_head_gate
        ? buffer_rsrc(g + (size_t)ce.start * H + (h & ~3), (uint32_t)L * (uint32_t)(H * 4))
        : rows(g, D, 4);
    const auto rK = qk_rows(k), rQ = qk_rows(q);
    const bool biased = gate_mode != 0 && dt_bias != nullptr;
    const auto rB = buffer_rsrc(biased ? dt_bias + (per_head_gate ? (size_t)(h & ~3) : (size_t)h * D) : g,
                                biased ? (per_head_gate ? 16 : D * 4) : 0);
    auto pick = [&](const float4 v) {
      const float x = hsub == 0 ? v.x : (hsub == 1 ? v.y : (hsub == 2 ? v.z : v.w));
      return per_head_gate ? f4(x) : v;
    };
    float4 gg[RPT];
    uint4 kk[K16], qq[K16];
    // byte offset of this thread's first row and the row stride
    const uint32_t gstride = (uint32_t)(per_head_gate ? H * 4 : H * D * 4);
    const uint32_t g0 = (uint32_t)(grp * RPT) * gstride + (per_head_gate ? 0u : (uint32_t)c4 * 4);
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      gg[i] = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(rG, g0 + (uint32_t)i * gstride, 0, NT_HINT));
#pragma unroll
    for (int i = 0; i < K16; ++i) {
      const int e = tid + i * NT, t = e / (D / IOV), c = (e % (D / IOV)) * IOV;
      const uint32_t off = (uint32_t)(t * HK * D + c) * (uint32_t)sizeof(IO);
      kk[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, NT_HINT));
      qq[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rQ, off, 0, NT_HINT));
    }
    // dt_bias of this thread's channels (zero without one)
    const float4 db = pick(__builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(rB, per_head_gate ? 0u : (uint32_t)c4 * 4, 0, 0)));
    if (per_head_gate) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) gg[i] = pick(gg[i]);
    }
    if (gate_mode != 0) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float4 x = gg[i] + db;
        float4 y;
        constexpr bool SAFE = GATE == 2;
        y = make_float4(gate1<SAFE>(x.x, rate, lower_bound), gate1<SAFE>(x.y, rate, lower_bound),
                        gate1<SAFE>(x.z, rate, lower_bound), gate1<SAFE>(x.w, rate, lower_bound));
        gg[i] = grp * RPT + i < L ? y : f4(0.f);  // rows past the sequence keep g = 0
      }
    }
    float4 acc = f4(0.f);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      acc = fma4(LOG2E, gg[i], acc);
      gg[i] = acc;
    }
    if (grp < NU) *reinterpret_cast<float4*>(sAA + grp * D + c4) = acc;
    float* sNrm = sAA + NU * D;  // [q rows, k rows] of inverse norms
    if (qk_l2norm) {
      // a row's GPR 16-byte groups sit in GPR consecutive lanes of one wave:
      // their sums of squares meet by a butterfly over those lanes
      constexpr int GPR = D / IOV;
#pragma unroll
      for (int i = 0; i < K16; ++i) {
        const int e = tid + i * NT;
        float sq = sumsq16<IO>(qq[i]), sk = sumsq16<IO>(kk[i]);
#pragma unroll
        for (int m = GPR / 2; m >= 1; m >>= 1) {
          sq += __shfl_xor(sq, m, 64);
          sk += __shfl_xor(sk, m, 64);
        }
        if (e < C * GPR && e % GPR == 0) {
          sNrm[e / GPR] = 1.f / sqrtf(sq + 1e-6f);
          sNrm[C + e / GPR] = 1.f / sqrtf(sk + 1e-6f);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < K16; ++i) {
      const int e = tid + i * NT, t = e / (D / IOV), c = (e % (D / IOV)) * IOV;
      if (e < C * (D / IOV)) {
        *reinterpret_cast<uint4*>(sK + iG(t, c)) = kk[i];
        *reinterpret_cast<uint4*>(sQ + iG(t, c)) = qq[i];
      }
    }
    __syncthreads();
    if (qk_l2norm && l < C) {
      rq_all = sNrm[l];
      rk_all = sNrm[C + l];
    }
    if (grp < NU) {
      float4 offs = f4(0.f);
      for (int g2 = 0; g2 < grp; ++g2) offs = offs + *reinterpret_cast<const float4*>(sAA + g2 * D + c4);
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        if (grp * RPT + i < C) *reinterpret_cast<float4*>(sG + iG(grp * RPT + i, c4)) = gg[i] + offs;
    }
  }
  __syncthreads();

  // Eight channels c0 .. c0 + 7 of row t, as fp32 (zero past D).
  auto row_io8 = [&](const IO* base, int t, int c0, float (&x)[8]) {
    if (c0 < D) {
      if (sizeof(IO) == 2) {
        lds8(reinterpret_cast<const bf16*>(base) + iG(t, c0), x);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(base + iG(t, c0));
        const float4 b = *reinterpret_cast<const float4*>(base + iG(t, c0) + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
  };
  auto row_g8 = [&](int t, int c0, float (&x)[8]) {
    if (c0 < D) {
      lds8(sG + iG(t, c0), x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
  };

  // ---- 3. A (strictly lower, from k; stored transposed) and Aq (lower, from
  // q) on the matrix cores.  Lane (lg, lr) of a unit owns row t = 16 I + lr
  // and channels 32 kt + 8 lg + j.  Both products share every exponential.
  //  - Off-diagonal blocks (J < I): exp(G_t - G_j) = exp(G_t - G_r)
  //    exp(G_r - G_j) through the block's first row r = 16 I, both <= 1.
  //  - Diagonal block: pairs in different 4-token sub-blocks factor through
  //    the first token r' of t's sub-block: three products (rows of
  //    sub-block s = 1..3 against the columns before r'), one tile each.
  //    Pairs inside one sub-block (and Aq's diagonal) follow in 3b.
  {
    auto store_tile = [&](int I, int J, f32x4 accA, f32x4 accQ, bool diag) {
      if (qk_l2norm) {  // rows t = 16 I + 4 lg + i, column j = 16 J + lr
        const float rkj = rk_of(16 * J + lr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * I + 4 * lg + i;
          accA[i] *= rk_of(t) * rkj;
          accQ[i] *= rq_of(t) * rkj;
        }
      }
      // keep, on the diagonal, rows of a later sub-block than the column only
      const bool keep = !diag || (lg > (lr >> 2));
      if (keep) {
        // A[t][j] -> sAA[j][t] (t = 16 I + 4 lg + i, j = 16 J + lr)
        *reinterpret_cast<f32x4*>(sAA + iA(16 * J + lr, 16 * I + 4 * lg)) = accA;
#pragma unroll
        for (int i = 0; i < 4; ++i) sAA[iA(16 * I + 4 * lg + i, 16 * J + lr)] = accQ[i];
      }
    };
    if (w < NB) {
      // diagonal unit, row block I = w.  Product p (reference token
      // 16 I + 4 p, p = 1..3) has its own accumulators; only the rows of
      // sub-block p keep it, and of those only the columns before the
      // reference, so nothing is masked: entries that mix other sub-blocks
      // (or overflow) are never stored.
      const int I = w, t = 16 * I + lr;
      f32x4 accA[3], accQ[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) accA[p] = accQ[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
      for (int kt = 0; kt < KTD; ++kt) {
        const int c0 = 32 * kt + 8 * lg;
        // the reference rows' G come from LDS, read as broadcasts (lanes
        // that share a reference row read one address): r' = the first
        // token of t's sub-block (4 lanes), and the first tokens 16 I + 4 sb
        // of sub-blocks 1 .. 3 (16 lanes)
        float k8[8], q8[8], g8[8], g0[8], gs[3][8];
        row_io8(sK, t, c0, k8);
        row_io8(sQ, t, c0, q8);
        row_g8(t, c0, g8);
        row_g8(t & ~3, c0, g0);
#pragma unroll
        for (int sb = 1; sb < 4; ++sb) row_g8(16 * I + 4 * sb, c0, gs[sb - 1]);
        float ra[8], rq[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = ex2(g8[j] - g0[j]);  // G_t - G_r' <= 0
          ra[j] = k8[j] * e;
          rq[j] = q8[j] * e;
        }
        const Frag fa = split8(ra), fq = split8(rq);
#pragma unroll
        for (int sb = 1; sb < 4; ++sb) {
          float b8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            b8[j] = k8[j] * ex2(gs[sb - 1][j] - g8[j]);  // G_ref - G_j <= 0 for kept columns
          const Frag fb = split8(b8);
          accA[sb - 1] = mma3(accA[sb - 1], fa, fb);
          accQ[sb - 1] = mma3(accQ[sb - 1], fq, fb);
        }
      }
      // accumulator rows 4 lg + i lie in sub-block lg (lg = 0 keeps nothing)
      const f32x4 A = lg == 1 ? accA[0] : (lg == 2 ? accA[1] : accA[2]);
      const f32x4 Q = lg == 1 ? accQ[0] : (lg == 2 ? accQ[1] : accQ[2]);
      store_tile(I, I, A, Q, true);
    } else {
      int I, J0, nJ;
      offdiag_group<NB>(w - NB, I, J0, nJ);
      if (nJ > 0) {
        const int t = 16 * I + lr;
        f32x4 accA[2], accQ[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) accA[u] = accQ[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KTD; ++kt) {
          const int c0 = 32 * kt + 8 * lg;
          // every LDS read of this step first (a wave with one column block
          // reads it twice), so that they are in flight together
          float k8[8], q8[8], g8[8], kj[2][8], gj[2][8];
          row_io8(sK, t, c0, k8);
          row_io8(sQ, t, c0, q8);
          row_g8(t, c0, g8);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int jr = 16 * (J0 + (u < nJ ? u : 0)) + lr;
            row_io8(sK, jr, c0, kj[u]);
            row_g8(jr, c0, gj[u]);
          }
          float gr[8], ra[8], rq[8];
          row_g8(16 * I, c0, gr);  // G at r = 16 I (a broadcast LDS read)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float e = ex2(g8[j] - gr[j]);
            ra[j] = k8[j] * e;
            rq[j] = q8[j] * e;
          }
          const Frag fa = split8(ra), fq = split8(rq);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            if (u < nJ) {
              float b8[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) b8[j] = kj[u][j] * ex2(gr[j] - gj[u][j]);
              const Frag fb = split8(b8);
              accA[u] = mma3(accA[u], fa, fb);
              accQ[u] = mma3(accQ[u], fq, fb);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (u < nJ) store_tile(I, J0 + u, accA[u], accQ[u], false);
      }
    }
  }
  // ---- 3b. pairs inside one 4-token sub-block (and Aq's diagonal),
  // elementwise, on the diagonal waves (they finish step 3 first): one
  // 16-lane row per sub-block, D / 16 consecutive channels per lane.  The 16
  // sums of a sub-block (6 of A, 6 of Aq, 4 diagonal) are reduced over the
  // row by a transposing butterfly: each step pairs lanes that differ in one
  // more index bit (mirror, half mirror, xor 2, xor 1), and each lane keeps
  // the half of its sums picked by that bit, so sum i ends in lane i.
  if (w < NB) {
    constexpr int CPL = D / 16;
    const int sb = tid >> 4, r = tid & 15, t0 = 4 * sb, c0 = CPL * r;
    float kk[4][CPL], qq[4][CPL], gg[4][CPL];
#pragma unroll
    for (int a2 = 0; a2 < 4; ++a2) {
      if constexpr (CPL == 8) {
        row_io8(sK, t0 + a2, c0, kk[a2]);
        row_io8(sQ, t0 + a2, c0, qq[a2]);
        row_g8(t0 + a2, c0, gg[a2]);
      } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          kk[a2][i] = to_f32(sK[iG(t0 + a2, c0 + i)]);
          qq[a2][i] = to_f32(sQ[iG(t0 + a2, c0 + i)]);
          gg[a2][i] = sG[iG(t0 + a2, c0 + i)];
        }
      }
    }
    float v[16];
    int n = 0;
#pragma unroll
    for (int a2 = 1; a2 < 4; ++a2)
#pragma unroll
      for (int b2 = 0; b2 < a2; ++b2, ++n) {
        float sa = 0.f, sq2 = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const float e = ex2(gg[a2][i] - gg[b2][i]) * kk[b2][i];
          sa = fmaf(kk[a2][i], e, sa);
          sq2 = fmaf(qq[a2][i], e, sq2);
        }
        v[n] = sa;
        v[6 + n] = sq2;
      }
#pragma unroll
    for (int a2 = 0; a2 < 4; ++a2) {
      float sd = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) sd = fmaf(qq[a2][i], kk[a2][i], sd);
      v[12 + a2] = sd;
    }
    butterfly_step<8, 0x140>(v, r & 8);  // partner 15 - r
    butterfly_step<4, 0x141>(v, r & 4);  // partner (r & 8) + 7 - (r & 7)
    butterfly_step<2, 0x4E>(v, r & 2);   // partner r ^ 2
    butterfly_step<1, 0xB1>(v, r & 1);   // partner r ^ 1
    // sum r: pairs n = r (A, stored transposed), n = r - 6 (Aq), diagonal r - 12
    const int m = r < 6 ? r : r - 6;
    const int a2 = 1 + (m >= 1) + (m >= 3), b2 = m - a2 * (a2 - 1) / 2;
    const int idx = r < 6 ? iA(t0 + b2, t0 + a2)
                          : (r < 12 ? iA(t0 + a2, t0 + b2) : iA(t0 + r - 12, t0 + r - 12));
    if (qk_l2norm) {  // row rt, column rj of the sum this lane holds
      // every shuffle runs on all lanes (a lane-dependent choice of which one
      // to run would leave source lanes inactive, and those read as zero)
      const int rt = r < 12 ? t0 + a2 : t0 + r - 12, rj = r < 12 ? t0 + b2 : rt;
      const float rkt = rk_of(rt), rqt = rq_of(rt), rkj = rk_of(rj);
      v[0] *= (r < 6 ? rkt : rqt) * rkj;
    }
    sAA[idx] = v[0];
  }
  __syncthreads();

  // Nothing is in flight on the vector memory counter here (every load so
  // far has been consumed); saying so resets the compiler's conservative
  // tracking, which would otherwise make the stores below wait for each other.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- 4. state-independent operands of the state pass
  // (scale Q e^G) as A fragments [NB][KTD]
  #pragma unroll
  for (int it_ = 0; it_ < (NB * KTD + NW - 1) / NW; ++it_) {
    const int tile = w + it_ * NW;
    if (tile >= NB * KTD) break;
    const int mt = tile / KTD, kt = tile % KTD, t = 16 * mt + lr, c0 = 32 * kt + 8 * lg;
    float x[8], g8[8];
    row_io8(sQ, t, c0, x);
    row_g8(t, c0, g8);
    const float sc = qk_l2norm ? scale * rq_of(t) : scale;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sc * x[j] * ex2(g8[j]);
    put_frag(Gm::Q_OFF + (uint32_t)tile * FRAG_BYTES, split8(x));
  }
  // (K e^{G_C - G})^T as A fragments [MTD][KTC]: rows = channels
  #pragma unroll
  for (int it_ = 0; it_ < (MTD * KTC + NW - 1) / NW; ++it_) {
    const int tile = w + it_ * NW;
    if (tile >= MTD * KTC) break;
    const int mt = tile / KTC, kt = tile % KTC, c = 16 * mt + lr;
    const float glast = sG[iG(C - 1, c)];
    // rows t0 + j share one swizzle base: the group index of (t0 + j, c) is
    // that of (t0, c) with its low three bits flipped by j (t0 % 8 == 0)
    constexpr int NG = D / 8;
    const int t0 = 32 * kt + 8 * lg;
    const int base = t0 * D + (c & 7), X = ((c >> 3) ^ t0) & (NG - 1);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = base + j * D + (((X ^ j) & (NG - 1)) << 3);
      x[j] = t0 + j < C ? to_f32(sK[idx]) * ex2(glast - sG[idx]) : 0.f;
    }
    if (qk_l2norm) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= rk_of(min(t0 + j, C - 1));
    }
    put_frag(Gm::KT_OFF + (uint32_t)tile * FRAG_BYTES, split8(x));
  }
  // scale Aq as A fragments [NB][KTC] (lower triangle of sAA)
  #pragma unroll
  for (int it_ = 0; it_ < (NB * KTC + NW - 1) / NW; ++it_) {
    const int tile = w + it_ * NW;
    if (tile >= NB * KTC) break;
    const int mt = tile / KTC, kt = tile % KTC, t = 16 * mt + lr;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = 32 * kt + 8 * lg + j;
      x[j] = (jj < C && jj <= t) ? scale * sAA[iA(t, jj)] : 0.f;
    }
    put_frag(Gm::AQ_OFF + (uint32_t)tile * FRAG_BYTES, split8(x));
  }
  if (tid < D)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ex2(sG[iG(C - 1, tid)])),
                                          buffer_rsrc(rec + Gm::GC_OFF, D * 4), (uint32_t)tid * 4, 0, 0);
  __syncthreads();  // q is dead: its space takes beta

  // ---- 5. K e^G in place of G (G no longer needed), in the plain row-major
  // layout that the column gathers of steps 8 and 10 read; beta into LDS
  if (tid < C) sB[tid] = (gate_mode != 0 && tid < L) ? sigmoid_fast(braw) : braw;
  {
    constexpr int G4 = (C * (D / 4) + NT - 1) / NT;
    float4 ke[G4];
#pragma unroll
    for (int i = 0; i < G4; ++i) {
      const int e = tid + i * NT, t = e / (D / 4), c = (e % (D / 4)) * 4;
      const float rk = qk_l2norm ? rk_of(min(t, C - 1)) : 1.f;
      if (e < C * (D / 4)) {
        const float4 kk = load4(sK + iG(t, c));
        const float4 gg = *reinterpret_cast<const float4*>(sG + iG(t, c));
        ke[i] = make_float4(kk.x * ex2(gg.x), kk.y * ex2(gg.y), kk.z * ex2(gg.z),
                            kk.w * ex2(gg.w));
        if (qk_l2norm) ke[i] = rk * ke[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < G4; ++i) {
      const int e = tid + i * NT, t = e / (D / 4), c = (e % (D / 4)) * 4;
      if (e < C * (D / 4)) *reinterpret_cast<float4*>(sG + iP(t, c)) = ke[i];
    }
  }
  __syncthreads();

  // v is only needed in step 9: its loads are issued here, past the steps
  // that need the most registers, and land while steps 6 - 8 run (raw io
  // bits; converted where they are used)
  constexpr int VPT = (C * (D / 4) + NT - 1) / NT;  // groups of four per thread
  typedef typename std::conditional<sizeof(IO) == 2, uint2, float4>::type Raw4;
  Raw4 vraw[VPT];
  {
    const auto rV = rows(v, D, (int)sizeof(IO));
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = tid + i * NT, t = e / (D / 4), c = (e % (D / 4)) * 4;
      const uint32_t off = (uint32_t)(t * H * D + c) * (uint32_t)sizeof(IO);
      if constexpr (sizeof(IO) == 2)
        vraw[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rV, off, 0, NT_HINT));
      else
        vraw[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rV, off, 0, NT_HINT));
    }
  }

  // ---- 6. X = (I + B A)^-1, B A strictly lower (A read transposed from the
  // upper triangle of sAA, X written to the lower one): 16 x 16 diagonal
  // blocks by forward substitution (one lane per column), then block rows.
  if (w < NB) {
    // Wave w inverts diagonal block w.  Lane (column cl = l % 16, quarter
    // p = l / 16) holds x_r of column cl for the rows r = p + 4 i.
    // Right-looking: once x_m is final it is broadcast from its lane, and
    // x_r -= (B A)[r][m] x_m for r > m; A[r][m] is read from sAA[m][r].
    const int b0 = 16 * w, cl = l & 15, p = l >> 4;
    float x[4], bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (p + 4 * i == cl) ? 1.f : 0.f;
      bb[i] = sB[b0 + p + 4 * i];
    }
#pragma unroll
    for (int m = 0; m < 15; ++m) {
      const float xm = __shfl(x[m >> 2], cl + 16 * (m & 3), 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = p + 4 * i;
        if (r > m) x[i] = fmaf(-bb[i] * sAA[iA(b0 + m, b0 + r)], xm, x[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = p + 4 * i;
      if (r >= cl) sAA[iA(b0 + r, b0 + cl)] = x[i];
    }
  }
  __syncthreads();  // also: k (step 5) is dead, its space becomes scratch
  // The off-diagonal blocks of X on the matrix cores.  (B A)[t][j] =
  // beta_t A[t][j] is read from A's transpose in the upper triangle of sAA, X
  // from the lower one (zero above the diagonal of a diagonal block).  An
  // accumulator tile passes through LDS scratch (sY) to become a B operand.
  // Helpers: the (B A) rows of block I against columns jb .. jb+31 of A
  // (below jend), and the X columns of block J over the same rows.
  auto ba_frag = [&](int I, int jb, int jend) {
    const float bt = sB[16 * I + lr];
    float a8[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = jb + 8 * lg + jj;
      a8[jj] = j < jend ? bt * sAA[iA(j, 16 * I + lr)] : 0.f;
    }
    return split8(a8);
  };
  auto x_frag = [&](int J, int jb, int jend) {
    float b8[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = jb + 8 * lg + jj;
      b8[jj] = (j < jend && j >= 16 * J + lr) ? sAA[iA(j, 16 * J + lr)] : 0.f;
    }
    return split8(b8);
  };
  // X_IJ = -X_II Y for the 16 x 16 tile Y held in accumulator layout
  auto x_times = [&](int I, int J, const f32x4& y, float* scratch) {
#pragma unroll
    for (int i = 0; i < 4; ++i) scratch[(4 * lg + i) * 16 + lr] = y[i];
    float a8[8], b8[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int m = 8 * lg + jj;
      a8[jj] = (lg < 2 && m <= lr) ? sAA[iA(16 * I + lr, 16 * I + m)] : 0.f;
      b8[jj] = lg < 2 ? scratch[m * 16 + lr] : 0.f;
    }
    const f32x4 x = mma3(f32x4{0.f, 0.f, 0.f, 0.f}, split8(a8), split8(b8));
#pragma unroll
    for (int i = 0; i < 4; ++i) sAA[iA(16 * I + 4 * lg + i, 16 * J + lr)] = -x[i];
  };
  if constexpr (NB == 4) {
    // Two levels of 2 x 2 block inversion (4 products on the critical path):
    //  A. X_10 and X_32: X_{I,I-1} = -X_II (B A)_{I,I-1} X_{I-1,I-1};
    //  B. the lower-left 32 x 32 block: T = (B A)_{[23],[01]} X_{[01],[01]},
    //     then X_{[23],[01]} = -X_{[23],[23]} T, one 16 x 16 tile per wave.
    if (w < 2) {
      const int I = 1 + 2 * w, J = I - 1;
      const f32x4 y = mma3(f32x4{0.f, 0.f, 0.f, 0.f}, ba_frag(I, 16 * J, 16 * I),
                           x_frag(J, 16 * J, 16 * I));
      x_times(I, J, y, sY + w * 256);
    }
    __syncthreads();
    float* sT = sY + 512;  // T tiles (I - 2) * 2 + J
    if (w < 4) {
      const int I = 2 + (w >> 1), J = w & 1;
      const f32x4 tt = mma3(f32x4{0.f, 0.f, 0.f, 0.f}, ba_frag(I, 16 * J, 32), x_frag(J, 16 * J, 32));
#pragma unroll
      for (int i = 0; i < 4; ++i) sT[w * 256 + (4 * lg + i) * 16 + lr] = tt[i];
    }
    __syncthreads();
    if (w < 4) {
      const int I = 2 + (w >> 1), J = w & 1, t = 16 * I + lr;
      float a8[8], b8[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int m = 32 + 8 * lg + jj;  // block K' = m / 16 of X_{I K'} and T_{K' J}
        a8[jj] = m <= t ? sAA[iA(t, m)] : 0.f;
        b8[jj] = sT[((m >> 4) - 2) * 512 + J * 256 + (m & 15) * 16 + lr];
      }
      const f32x4 x = mma3(f32x4{0.f, 0.f, 0.f, 0.f}, split8(a8), split8(b8));
#pragma unroll
      for (int i = 0; i < 4; ++i) sAA[iA(16 * I + 4 * lg + i, 16 * J + lr)] = -x[i];
    }
    __syncthreads();
  } else {
    // block rows I = 1 .. NB - 1 in turn, block (I, J) on wave J < I:
    //   Y_J = sum_{K=J}^{I-1} (B A)_{IK} X_{KJ},   X_IJ = -X_II Y_J
#pragma unroll
    for (int I = 1; I < NB; ++I) {
      if (w < I) {
        const int J = w;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j0 = 0; j0 < 16 * NB; j0 += 32) {
          const int jb = 16 * J + j0;
          if (jb >= 16 * I) break;
          y = mma3(y, ba_frag(I, jb, 16 * I), x_frag(J, jb, 16 * I));
        }
        x_times(I, J, y, sY + w * 256);
      }
      __syncthreads();
    }
  }

  // ---- 7. M = X diag(beta) as split A fragments [NB][KTC] (over k), shared
  // by all waves
  #pragma unroll
  for (int it_ = 0; it_ < (NB * KTC + NW - 1) / NW; ++it_) {
    const int tile = w + it_ * NW;
    if (tile >= NB * KTC) break;
    const int mt = tile / KTC, kt = tile % KTC, t = 16 * mt + lr;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = 32 * kt + 8 * lg + j;
      x[j] = (jj < C && jj <= t) ? sAA[iA(t, jj)] * sB[jj] : 0.f;
    }
    const Frag f = split8(x);
    sMf[tile * 128 + l] = f.hi;
    sMf[tile * 128 + 64 + l] = f.lo;
  }
  __syncthreads();

  // ---- 8. W = M (K e^G), 32 rows at a time staged in LDS (over sAA) and
  // written out as A fragments; a wave owns 16-channel column tiles and
  // splits their B fragments once, before the first half
  constexpr int NTW = (MTD + NW - 1) / NW;  // column tiles per wave
  Frag fbw[NTW][KTC];
  #pragma unroll
  for (int it_ = 0; it_ < NTW; ++it_) {
    const int nt = w + it_ * NW;
    if (nt >= MTD) break;
#pragma unroll
    for (int kt = 0; kt < KTC; ++kt) {
      float b8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = 32 * kt + 8 * lg + j;
        b8[j] = jj < C ? sG[iP(jj, 16 * nt + lr)] : 0.f;
      }
      fbw[it_][kt] = split8(b8);
    }
  }
  for (int half = 0; half < (NB + 1) / 2; ++half) {
    #pragma unroll
    for (int it_ = 0; it_ < NTW; ++it_) {
      const int nt = w + it_ * NW;
      if (nt >= MTD) break;
      const Frag (&fb)[KTC] = fbw[it_];
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int mt = 2 * half + m2;
        if (mt < NB) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kt = 0; kt < KTC; ++kt) {
            if (32 * kt > 16 * mt + 15) break;  // X is lower triangular
            Frag fa;
            fa.hi = sMf[(mt * KTC + kt) * 128 + l];
            fa.lo = sMf[(mt * KTC + kt) * 128 + 64 + l];
            acc = mma3(acc, fa, fb[kt]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sW[iW(16 * m2 + 4 * lg + i, 16 * nt + lr)] = acc[i];
        }
      }
    }
    __syncthreads();
    #pragma unroll
    for (int it_ = 0; it_ < (2 * KTD + NW - 1) / NW; ++it_) {
      const int tile = w + it_ * NW;
      if (tile >= 2 * KTD) break;
      const int m2 = tile / KTD, kt = tile % KTD, mt = 2 * half + m2;
      if (mt < NB) {
        const int c0 = 32 * kt + 8 * lg;
        float x[8];
        if (c0 < D) {
          lds8(sW + iW(16 * m2 + lr, c0), x);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = 0.f;
        }
        put_frag(Gm::W_OFF + (uint32_t)(mt * KTD + kt) * FRAG_BYTES, split8(x));
      }
    }
    __syncthreads();
  }

  // ---- 9. V (fetched at the start) in place of K e^G
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int e = tid + i * NT, t = e / (D / 4), c = (e % (D / 4)) * 4;
    if (e < C * (D / 4)) {
      float4 x;
      if constexpr (sizeof(IO) == 2)  // bf16 pairs: element 2j in the low half of word j
        x = make_float4(__uint_as_float(vraw[i].x << 16), __uint_as_float(vraw[i].x & 0xffff0000u),
                        __uint_as_float(vraw[i].y << 16), __uint_as_float(vraw[i].y & 0xffff0000u));
      else
        x = vraw[i];
      *reinterpret_cast<float4*>(sG + iP(t, c)) = x;
    }
  }
  __syncthreads();

  // ---- 10. U = M V, stored as accumulator tiles [NB][MTD].  A bf16 V is
  // exact in bf16, so its lo part is zero and that product is skipped.
  #pragma unroll
  for (int it_ = 0; it_ < (MTD + NW - 1) / NW; ++it_) {
    const int nt = w + it_ * NW;
    if (nt >= MTD) break;
    Frag fb[KTC];
#pragma unroll
    for (int kt = 0; kt < KTC; ++kt) {
      float b8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = 32 * kt + 8 * lg + j;
        b8[j] = jj < C ? sG[iP(jj, 16 * nt + lr)] : 0.f;
      }
      fb[kt] = split8(b8);
    }
#pragma unroll
    for (int mt = 0; mt < NB; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KTC; ++kt) {
        if (32 * kt > 16 * mt + 15) break;
        Frag fa;
        fa.hi = sMf[(mt * KTC + kt) * 128 + l];
        fa.lo = sMf[(mt * KTC + kt) * 128 + 64 + l];
        if (sizeof(IO) == 2) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.lo, fb[kt].hi, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.hi, fb[kt].hi, acc, 0, 0, 0);
        } else {
          acc = mma3(acc, fa, fb[kt]);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, acc), buffer_rsrc(rec + Gm::U_OFF + (size_t)(mt * MTD + nt) * 1024, 1024),
          lane16, 0, NT_HINT);
    }
  }
}

// ------------------------------------------------------------------ state

template <typename IO, int D, int C, int VT>
struct StateSmem {
  static constexpr int SK = (D < 32 ? 32 : D) + 8;        // S^T row: channels (+pad)
  static constexpr int DK = Geom<D, C>::KTC * 32 + 8;     // D^T row: tokens (+pad)
  static constexpr size_t S_BYTES = (size_t)VT * SK * 2;  // one bf16 plane
  static constexpr size_t D_BYTES = (size_t)VT * DK * 2;
  static constexpr size_t O_BYTES = (size_t)16 * VT * sizeof(IO);  // one wave's O tile
  static constexpr size_t S_OFF = 0;                       // [hi, lo]
  static constexpr size_t D_OFF = 2 * S_BYTES;             // [hi, lo]
  static constexpr size_t O_OFF = D_OFF + 2 * D_BYTES;     // [4 waves]
  static constexpr size_t TOTAL = O_OFF + 4 * O_BYTES;
};

// Per-wave operands of one chunk that the state pass reads from the workspace.
template <int D, int C, int VT>
struct StateOps {
  typedef Geom<D, C> Gm;
  static constexpr int NTV = VT / 16, KTC = Gm::KTC, KTD = Gm::KTD;
  static constexpr int MS = (Gm::MTD + 3) / 4;  // state row tiles per wave
  Frag w[KTD], q[KTD];     // row tile mt = wave of W and scale Q e^G
  f32x4 u[NTV];            // U tiles of this V tile
  Frag aq[KTC];            // scale Aq, row tile mt
  Frag kt[MS][KTC];        // (K e^{G_C-G})^T, row tiles ms = wave + 4 i
  f32x4 gc[MS];            // e^{G_C} of the rows of those tiles
};

// One work unit (see Unit) on one V tile vt of D / VT (MAP: one column tile
// vt of the 2 D columns of [M | B]).
template <typename IO, int D, int C, int VT, bool MAP>
__device__ __forceinline__ void state_unit(
    char* smem, const SeqInfo* __restrict__ seqs, const Unit& un, int h, int vt,
    const char* __restrict__ recs, int ncb, int H, const float* __restrict__ h0,
    float* __restrict__ ht, IO* __restrict__ o, float* __restrict__ snaps, int64_t snap_rows,
    int snap_interval, float* __restrict__ starts, float* __restrict__ maps) {
  typedef Geom<D, C> Gm;
  typedef StateSmem<IO, D, C, VT> Sm;
  typedef StateOps<D, C, VT> Ops;
  constexpr int NV = D / VT, NTV = VT / 16, NB = Gm::NB, KTC = Gm::KTC, KTD = Gm::KTD;
  constexpr int MTD = Gm::MTD, MS = Ops::MS;
  constexpr int SK = Sm::SK, DK = Sm::DK;
  constexpr int NTILE = MAP ? 2 * NV : NV;  // workgroups per (unit, head)
  bf16* sDh = reinterpret_cast<bf16*>(smem + Sm::D_OFF);
  bf16* sDl = reinterpret_cast<bf16*>(smem + Sm::D_OFF + Sm::D_BYTES);

  // workgroup-uniform values as scalars, so that every branch on them is
  // uniform and the chunk table is read through scalar loads
  const int n = __builtin_amdgcn_readfirstlane(un.seq);
  const int flags = __builtin_amdgcn_readfirstlane(un.flags);
  const int in_slot = __builtin_amdgcn_readfirstlane(un.in_slot);
  const int out_slot = __builtin_amdgcn_readfirstlane(un.out_slot);
  if (!MAP && flags == 0) return;  // a wave this sequence does not reach
  const int tid = threadIdx.x, l = tid & 63, lg = l >> 4, lr = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // When every wave owns a chunk row tile and the same number of state row
  // tiles (the usual D and C), these tests are compile-time true: no branch
  // then separates the operand loads, and the wait counts the compiler places
  // for them stay exact, so the next chunk's loads are never waited for.
  constexpr bool ALL_MT = NB >= 4, ALL_MS = MTD % 4 == 0;
  const bool has_mt = ALL_MT || w < NB;
  const int mt = w;
  IO* sO = reinterpret_cast<IO*>(smem + Sm::O_OFF + w * Sm::O_BYTES);

  // zero the LDS padding once (k positions beyond D or C stay zero)
  for (int e = tid; e < (int)(Sm::TOTAL / 4); e += NTHREADS) reinterpret_cast<int*>(smem)[e] = 0;

  // state tiles owned by this wave: ms = w + 4 i, all NTV column tiles.  A
  // map starts from [I | 0]; a later segment from its start slot; a first
  // segment from h0 (or zeros).
  const float* init = nullptr;
  if (!MAP) {
    if (flags & UNIT_FROM_START)
      init = starts + ((size_t)in_slot * H + h) * D * D;
    else if (h0 != nullptr)
      init = h0 + ((size_t)n * H + h) * D * D;
  }
  f32x4 S[MS][NTV];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int ms = w + 4 * i;
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * ms + 4 * lg + e, col = vt * VT + 16 * nt + lr;
        float x = 0.f;
        if (MAP)
          x = row == col ? 1.f : 0.f;
        else if (init != nullptr && (ALL_MS || ms < MTD))
          x = init[row * D + col];
        S[i][nt][e] = x;
      }
    }
  }

  // the sequence's tokens and first chunk, from the plan (disjoint clamped
  // ranges, so no chunk index passes the workspace's chunk count)
  const SeqInfo si = seqs[n];
  const int seq_start = __builtin_amdgcn_readfirstlane(si.lo);
  const int seq_end = __builtin_amdgcn_readfirstlane(si.hi);
  // chunk ch of the unit is chunk r_begin + (ch - c_begin) of its sequence
  const int r_shift = __builtin_amdgcn_readfirstlane(un.r_begin) -
                      __builtin_amdgcn_readfirstlane(un.c_begin);
  const int c_begin = __builtin_amdgcn_readfirstlane(un.c_begin);
  const int c_last = min(ncb, __builtin_amdgcn_readfirstlane(un.c_end));
  // snapshot rows of this sequence follow those of sequences 0 .. n-1
  const int snap_base = __builtin_amdgcn_readfirstlane(si.snap_base);
  // U's column tile (a map's M columns have no U: D = -W S there)
  const bool has_u = !MAP || vt >= NV;
  const int ut = MAP ? vt - NV : vt;
  // Every operand of a chunk is loaded unconditionally (including Aq tiles
  // above the diagonal, which are never multiplied), so the loads form one
  // straight block.
  const uint32_t lane16 = (uint32_t)l * 16u;
  auto rsrc_of = [&](int ch) {
    return buffer_rsrc(recs + ((size_t)h * ncb + ch) * Gm::REC, (uint32_t)Gm::REC);
  };
  // The operand set of a chunk is fetched in four parts, so that the fetch
  // of chunk i+1 can be spread over the phases of chunk i.
  auto load_w = [&](Ops& ops, __amdgpu_buffer_rsrc_t r) {
    if (has_mt) {
#pragma unroll
      for (int kt = 0; kt < KTD; ++kt)
        ops.w[kt] = buffer_frag(r, lane16, Gm::W_OFF + (mt * KTD + kt) * FRAG_BYTES);
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt)
        ops.u[nt] = has_u ? buffer_f32x4(r, lane16, Gm::U_OFF + ((mt * MTD + ut * NTV + nt) * 64) * 16)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto load_kt = [&](Ops& ops, __amdgpu_buffer_rsrc_t r) {
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int ms = w + 4 * i;
      if (ALL_MS || ms < MTD) {
        ops.gc[i] = buffer_f32x4(r, (uint32_t)lg * 16u, Gm::GC_OFF + 64 * ms);
#pragma unroll
        for (int kt = 0; kt < KTC; ++kt)
          ops.kt[i][kt] = buffer_frag(r, lane16, Gm::KT_OFF + (ms * KTC + kt) * FRAG_BYTES);
      }
    }
  };
  auto load_q = [&](Ops& ops, __amdgpu_buffer_rsrc_t r) {
    if (!MAP && has_mt) {
#pragma unroll
      for (int kt = 0; kt < KTD; ++kt)
        ops.q[kt] = buffer_frag(r, lane16, Gm::Q_OFF + (mt * KTD + kt) * FRAG_BYTES);
    }
  };
  auto load_aq = [&](Ops& ops, __amdgpu_buffer_rsrc_t r) {
    if (!MAP && has_mt) {
#pragma unroll
      for (int kt = 0; kt < KTC; ++kt)
        ops.aq[kt] = buffer_frag(r, lane16, Gm::AQ_OFF + (mt * KTC + kt) * FRAG_BYTES);
    }
  };
  auto load = [&](Ops& ops, int ch) {
    const __amdgpu_buffer_rsrc_t r = rsrc_of(ch);
    load_w(ops, r);
    load_kt(ops, r);
    load_q(ops, r);
    load_aq(ops, r);
  };

  // One chunk.  The carried chain is S -> P = W S -> D = U - P -> S update;
  // the read-out O = (Q e^G) S + Aq D follows the update.  Each phase first
  // reads all of its LDS fragments, then issues its MFMAs back to back; the
  // entering S and D fragments stay in registers for the read-out.
  bf16* sSh = reinterpret_cast<bf16*>(smem + Sm::S_OFF);
  bf16* sSl = reinterpret_cast<bf16*>(smem + Sm::S_OFF + Sm::S_BYTES);
  // L2 prefetch two chunks ahead: the NTILE workgroups of a (unit, head)
  // each touch one word in every NTILE-th 128-byte line of the record, so the
  // operand loads of that chunk, issued one chunk later, hit L2.  The words
  // are read into registers that are consumed one chunk after that, when the
  // loads have long completed.
  constexpr int LINES = (int)(Gm::REC / 128);
  constexpr int NPF = (LINES + NTILE * NTHREADS - 1) / (NTILE * NTHREADS);
  int pf[NPF];
#pragma unroll
  for (int i = 0; i < NPF; ++i) pf[i] = 0;
  auto prefetch = [&](int ch) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) asm volatile("" ::"v"(pf[i]));
    const __amdgpu_buffer_rsrc_t r = rsrc_of(min(ch + 2, c_last - 1));
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int line = vt + NTILE * (tid + NTHREADS * i);
      // out-of-range offsets read as zero (the buffer bound is the record)
      pf[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)line * 128u, 0, 0);
    }
  };

  auto process = [&](Ops& ops, int ch) {
    const __amdgpu_buffer_rsrc_t rn = rsrc_of(min(ch + 1, c_last - 1));
    // -- 1. S^T (hi, lo) into LDS
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int ms = w + 4 * i;
      if (ALL_MS || ms < MTD) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
          bf16x4v hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16 hh = (bf16)S[i][nt][e];
            hi[e] = hh;
            lo[e] = (bf16)(S[i][nt][e] - (float)hh);
          }
          const int at = (16 * nt + lr) * SK + 16 * ms + 4 * lg;
          *reinterpret_cast<bf16x4v*>(sSh + at) = hi;
          *reinterpret_cast<bf16x4v*>(sSl + at) = lo;
        }
      }
    }
    __syncthreads();

    // -- 2. row tile mt = w: P = W S, D = U - P into LDS
    Frag fs[KTD][NTV];
    if (has_mt) {
#pragma unroll
      for (int kt = 0; kt < KTD; ++kt)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
          const int at = (16 * nt + lr) * SK + 32 * kt + 8 * lg;
          fs[kt][nt].hi = *reinterpret_cast<const bf16x8*>(sSh + at);
          fs[kt][nt].lo = *reinterpret_cast<const bf16x8*>(sSl + at);
        }
      f32x4 P[NTV];
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) P[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KTD; ++kt)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) P[nt] = mma3(P[nt], ops.w[kt], fs[kt][nt]);
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        bf16x4v hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = ops.u[nt][e] - P[nt][e];
          const bf16 hh = (bf16)d;
          hi[e] = hh;
          lo[e] = (bf16)(d - (float)hh);
        }
        const int at = (16 * nt + lr) * DK + 16 * mt + 4 * lg;
        *reinterpret_cast<bf16x4v*>(sDh + at) = hi;
        *reinterpret_cast<bf16x4v*>(sDl + at) = lo;
      }
    }
    __syncthreads();

    // -- 3. S = Diag(e^{G_C}) S + (K e^{G_C - G})^T D
    Frag fd[KTC][NTV];
#pragma unroll
    for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        const int at = (16 * nt + lr) * DK + 32 * kt + 8 * lg;
        fd[kt][nt].hi = *reinterpret_cast<const bf16x8*>(sDh + at);
        fd[kt][nt].lo = *reinterpret_cast<const bf16x8*>(sDl + at);
      }
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int ms = w + 4 * i;
      if (ALL_MS || ms < MTD) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[i][nt][e] *= ops.gc[i][e];
#pragma unroll
        for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt) S[i][nt] = mma3(S[i][nt], ops.kt[i][kt], fd[kt][nt]);
      }
    }
    // W and U of this chunk are dead: fetch the next ones between the MFMAs
    load_w(ops, rn);
    interleave_loads<3 * MS * KTC * NTV, 2 * KTD + NTV>();

    // -- 4. O = (scale Q e^G) S + (scale Aq) D for row tile mt
    // (K e^{G_C-G} and e^{G_C} of this chunk are dead: every wave that owns
    // state rows fetches the next ones, spread between the MFMAs below)
    load_kt(ops, rn);
    if (!MAP && has_mt) {
      f32x4 O[NTV];
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) O[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KTD; ++kt)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) O[nt] = mma3(O[nt], ops.q[kt], fs[kt][nt]);
      interleave_loads<3 * KTD * NTV, MS * (2 * KTC + 1)>();
#pragma unroll
      for (int kt = 0; kt < KTC; ++kt) {
        if (32 * kt > 16 * mt + 15) break;  // Aq is lower triangular (uniform)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) O[nt] = mma3(O[nt], ops.aq[kt], fd[kt][nt]);
      }
      load_q(ops, rn);
      load_aq(ops, rn);
      // stage the 16 x VT tile in this wave's LDS slot, then 16-byte stores
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sO[(4 * lg + e) * VT + 16 * nt + lr] = from_f32<IO>(O[nt][e]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int c_start = seq_start + (ch + r_shift) * C;
      const int c_len = min(C, seq_end - c_start);
      constexpr int ROW16 = VT * (int)sizeof(IO) / 16;  // 16-byte pieces per row
#pragma unroll
      for (int p = l; p < 16 * ROW16; p += 64) {
        const int r = p / ROW16, c16 = p % ROW16;
        const int t = 16 * mt + r;
        const uint4 val = *reinterpret_cast<const uint4*>(sO + r * VT + c16 * (16 / sizeof(IO)));
        if (t < c_len)
          *reinterpret_cast<uint4*>(o + ((int64_t)(c_start + t) * H + h) * D + vt * VT +
                                    c16 * (16 / sizeof(IO))) = val;
      }
    }
    // chunk-boundary snapshot: the state after this chunk, when the chunk
    // ends a whole multiple of snap_interval tokens into the sequence
    if (!MAP && snaps != nullptr) {
      const int end_tok = (ch + r_shift + 1) * C;
      const int64_t row = (int64_t)snap_base + end_tok / snap_interval - 1;
      if (end_tok <= seq_end - seq_start && end_tok % snap_interval == 0 && row < snap_rows) {
        float* P = snaps + (row * H + h) * D * D;
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          const int ms = w + 4 * i;
          if (ALL_MS || ms < MTD) {
#pragma unroll
            for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                __builtin_nontemporal_store(
                    S[i][nt][e], P + (16 * ms + 4 * lg + e) * D + vt * VT + 16 * nt + lr);
          }
        }
      }
    }
    // the L2 prefetch goes last: the wave's wait counter drains in issue
    // order, so a fetch of the next chunk's operands never waits for it
    prefetch(ch);
  };

  // One operand set in registers: each part is refetched for chunk i+1 as
  // soon as chunk i has used it, so every fetch has about one chunk period
  // to arrive (the last fetch repeats the last chunk and goes unused).
  // The initial state's loads complete here: otherwise the compiler's wait
  // analysis, which merges this path with the loop's back edge, can make the
  // top of every chunk wait for all outstanding loads.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  Ops ops;
  if (c_begin < c_last) load(ops, c_begin);
  __syncthreads();
  for (int ch = c_begin; ch < c_last; ++ch) process(ops, ch);

  // the final state: ht (the whole sequence or its last segment), the next
  // segment's start slot, or the map slot.  A map [M | B] (D rows, 2 D
  // columns per head) is stored in 4-column tiles, element (i, j) at
  // ((j / 4) D + i) 4 + j % 4, so that the scan's row-per-thread reads of
  // four columns are contiguous across threads.
  float* dst = nullptr;
  if (MAP) {
    float* mp = maps + ((size_t)out_slot * H + h) * D * 2 * D;
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int ms = w + 4 * i;
      if (ALL_MS || ms < MTD) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * ms + 4 * lg + e, col = vt * VT + 16 * nt + lr;
            mp[((size_t)(col >> 2) * D + row) * 4 + (col & 3)] = S[i][nt][e];
          }
      }
    }
  } else if (flags & UNIT_WRITE_NEXT) {
    dst = starts + ((size_t)out_slot * H + h) * D * D;
  } else if ((flags & UNIT_WRITE_HT) && ht != nullptr) {
    dst = ht + ((size_t)n * H + h) * D * D;
  }
  if (dst != nullptr) {
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int ms = w + 4 * i;
      if (ALL_MS || ms < MTD) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dst[(size_t)(16 * ms + 4 * lg + e) * D + vt * VT + 16 * nt + lr] = S[i][nt][e];
      }
    }
  }
}

// The state pass over a list of units: blocks 0 .. 8 * NV * ceil(H nu / 8)
// - 1 take the units of `units` (nu = *n_units of them), each on its NV V
// tiles; with maps, the blocks after them take the map units (*n_maps), each
// on the 2 NV column tiles of [M | B].  Block ids are XCD-aware: the tiles
// of one (unit, head) get ids congruent mod 8, so they share one L2.
template <typename IO, int D, int C, int VT>
__global__ __launch_bounds__(NTHREADS, 1) void state_kernel(
    const SeqInfo* __restrict__ seqs, const Unit* __restrict__ units,
    const int* __restrict__ n_units, int units_max, const Unit* __restrict__ map_units,
    const int* __restrict__ n_maps, const char* __restrict__ recs, int ncb, int H,
    const float* __restrict__ h0, float* __restrict__ ht, IO* __restrict__ o,
    float* __restrict__ snaps, int64_t snap_rows, int snap_interval, float* __restrict__ starts,
    float* __restrict__ maps) {
  typedef StateSmem<IO, D, C, VT> Sm;
  constexpr int NV = D / VT;
  __shared__ __align__(16) char smem[Sm::TOTAL];
  const int norm_blocks = (H * units_max + 7) / 8 * 8 * NV;
  int b = blockIdx.x;
  if (b < norm_blocks) {
    const int vt = (b / 8) % NV;
    const int u = (b / (8 * NV)) * 8 + (b % 8);
    if (u >= __builtin_amdgcn_readfirstlane(*n_units) * H) return;
    state_unit<IO, D, C, VT, false>(smem, seqs, units[u / H], u % H, vt, recs, ncb, H, h0, ht, o,
                                    snaps, snap_rows, snap_interval, starts, maps);
  } else {
    b -= norm_blocks;
    const int vt = (b / 8) % (2 * NV);
    const int u = (b / (16 * NV)) * 8 + (b % 8);
    if (map_units == nullptr || u >= __builtin_amdgcn_readfirstlane(*n_maps) * H) return;
    state_unit<IO, D, C, VT, true>(smem, seqs, map_units[u / H], u % H, vt, recs, ncb, H, h0, ht,
                                   o, snaps, snap_rows, snap_interval, starts, maps);
  }
}

// Start states of the later segments of every cut sequence: start(p) of
// segment p + 1 = M_p start(p - 1) + B_p for the middle segments p = 1 ..
// nseg - 2, in order (start slot 0 of the sequence holds the first segment's
// final state).  One workgroup per (sequence, head, group of 4 columns), one
// thread per row; fp32 throughout.  The maps' 4-column tiles make a wave's
// reads of 16-byte row pieces contiguous.  A thread holds its row of M_p in
// registers, and each 16-byte piece of the next map's row is requested as
// soon as this step has used that piece: the loads of step p + 1 are in
// flight while step p computes, so the serial chain pays the load latency
// once instead of at every step.
template <int D>
__global__ __launch_bounds__(D) void scan_kernel(const SeqInfo* __restrict__ seqs, int N, int H,
                                                 int C, int seg_len,
                                                 const float* __restrict__ maps,
                                                 float* __restrict__ starts) {
  __shared__ float4 sS[D];
  const int groups = D / 4;
  const int b = blockIdx.x;
  const int cg = b % groups, h = (b / groups) % H, n = b / (groups * H);
  if (n >= N) return;
  const SeqInfo si = seqs[n];
  const int nch = (si.hi - si.lo + C - 1) / C;
  const int nseg = nch > seg_len ? (nch + seg_len - 1) / seg_len : 1;
  if (nseg < 3) return;
  const int i = threadIdx.x;
  // row i of map p, [M_p | B_p] in 4-column tiles: columns 4 j4 .. 4 j4 + 3
  // of row i at float4 j4 D + i
  auto map_row = [&](int p) {
    return reinterpret_cast<const float4*>(maps + ((size_t)(si.map_slot + p - 1) * H + h) * D * 2 * D) + i;
  };
  float4 m[D / 4];
  float4 bp;
  {
    const float4* M = map_row(1);
#pragma unroll
    for (int j4 = 0; j4 < D / 4; ++j4) m[j4] = M[j4 * D];
    bp = M[(D / 4 + cg) * D];
  }
  float4 x = *reinterpret_cast<const float4*>(starts + (((size_t)si.start_slot * H + h) * D + i) * D +
                                              4 * cg);
  // L2 prefetch two maps ahead: the groups workgroups of a (sequence, head)
  // each touch one word of every groups-th 128-byte line of that map; the
  // word is consumed a step later, when it has long arrived
  constexpr int LINES = D * 2 * D * 4 / 128;
  constexpr int NPF = (LINES / groups + D - 1) / D;
  int pf[NPF];
#pragma unroll
  for (int q = 0; q < NPF; ++q) pf[q] = 0;
  for (int p = 1; p <= nseg - 2; ++p) {
#pragma unroll
    for (int q = 0; q < NPF; ++q) asm volatile("" ::"v"(pf[q]));
    {
      const int pp = p + 2 <= nseg - 2 ? p + 2 : nseg - 2;
      const int* mw = reinterpret_cast<const int*>(
          maps + ((size_t)(si.map_slot + pp - 1) * H + h) * D * 2 * D);
#pragma unroll
      for (int q = 0; q < NPF; ++q) {
        // unconditional (a line past the map repeats line 0): a select on
        // the loaded word would make the wave wait for it here
        const int line = cg + groups * (i + D * q);
        pf[q] = mw[(line < LINES ? line : 0) * 32];
      }
    }
    sS[i] = x;
    __syncthreads();
    // the next map's row (the last step re-reads its own: never used)
    const float4* Mn = map_row(p + 1 <= nseg - 2 ? p + 1 : p);
    // four partial sums (j4 mod 4), so that no single fma chain runs the
    // length of the row
    float4 acc[4] = {bp, f4(0.f), f4(0.f), f4(0.f)};
    bp = Mn[(D / 4 + cg) * D];
#pragma unroll
    for (int j4 = 0; j4 < D / 4; ++j4) {
      const float4 mm = m[j4];
      float4& a = acc[j4 & 3];
      a = fma4(mm.x, sS[4 * j4], a);
      a = fma4(mm.y, sS[4 * j4 + 1], a);
      a = fma4(mm.z, sS[4 * j4 + 2], a);
      a = fma4(mm.w, sS[4 * j4 + 3], a);
      m[j4] = Mn[j4 * D];
    }
    __syncthreads();
    x = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    *reinterpret_cast<float4*>(starts + (((size_t)(si.start_slot + p) * H + h) * D + i) * D +
                               4 * cg) = x;
  }
}

// ----------------------------------------------------------------- launch

// V tile of the state pass: every tile's workgroup loads the chunk's full
// W, Q e^G, K e^{G_C-G} and Aq, so wider tiles cut the replicated operand
// traffic (per-CU load bandwidth) at the cost of fewer, busier workgroups.
template <int D>
constexpr int state_vt() { return D >= 32 ? 32 : D; }

// The second stream of the wave schedule: one per device, created on first
// use (non-blocking, default priority), with a pool of events.  Events are
// only borrowed while a call enqueues its work: a wait binds to the record
// that precedes it in enqueue order, so reusing an event in a later call
// cannot disturb an earlier call's waits.
struct AuxStream {
  hipStream_t stream = nullptr;
  std::vector<hipEvent_t> free_events;
};
constexpr int kMaxDevices = 64;
std::mutex aux_mu;
AuxStream aux_streams[kMaxDevices];

hipError_t aux_acquire(int n_events, hipStream_t& aux, std::vector<hipEvent_t>& ev) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(aux_mu);
  AuxStream& a = aux_streams[dev];
  if (a.stream == nullptr &&
      (e = hipStreamCreateWithFlags(&a.stream, hipStreamNonBlocking)) != hipSuccess)
    return e;
  aux = a.stream;
  ev.clear();
  while ((int)ev.size() < n_events) {
    hipEvent_t x;
    if (!a.free_events.empty()) {
      x = a.free_events.back();
      a.free_events.pop_back();
    } else if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) {
      for (hipEvent_t y : ev) a.free_events.push_back(y);
      ev.clear();
      return e;
    }
    ev.push_back(x);
  }
  return hipSuccess;
}

void aux_release(const std::vector<hipEvent_t>& ev) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(aux_mu);
  for (hipEvent_t x : ev) aux_streams[dev].free_events.push_back(x);
}

// Stream of the caller's device: the aux stream must belong to the same
// device as `st` (the current device); a stream of another device runs the
// schedule on that one stream.
bool stream_on_current_device(hipStream_t st) {
  if (st == nullptr) return true;
  int cur = 0;
  hipDevice_t dev = 0;
  return hipGetDevice(&cur) == hipSuccess && hipStreamGetDevice(st, &dev) == hipSuccess &&
         dev == cur;
}

// A stream being captured into a graph keeps the whole schedule: the second
// stream is used only for eager work.
bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return st != nullptr && (hipStreamIsCapturing(st, &cs) != hipSuccess ||
                           cs != hipStreamCaptureStatusNone);
}

template <typename IO, int D, int C>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  typedef Geom<D, C> Gm;
  constexpr int VT = state_vt<D>();
  constexpr int NV = D / VT;
  const WsLayout ws = ws_layout(a.T, a.N, a.H, D, C, Gm::REC);
  const StateCut& cut = ws.cut;
  char* base = reinterpret_cast<char*>(a.ws);
  ChunkEntry* table = reinterpret_cast<ChunkEntry*>(base + ws.table_off);
  SeqInfo* seqs = reinterpret_cast<SeqInfo*>(base + ws.seq_off);
  Unit* units_a = reinterpret_cast<Unit*>(base + ws.unit_a_off);
  Unit* units_m = reinterpret_cast<Unit*>(base + ws.unit_m_off);
  Unit* units_c = reinterpret_cast<Unit*>(base + ws.unit_c_off);
  Unit* units_w = reinterpret_cast<Unit*>(base + ws.unit_w_off);
  int* counts = reinterpret_cast<int*>(base + ws.count_off);
  int* wave_off = reinterpret_cast<int*>(base + ws.wave_off);
  char* recs = base + ws.rec_off;
  float* starts = reinterpret_cast<float*>(base + ws.start_off);
  float* maps = reinterpret_cast<float*>(base + ws.map_off);
  auto mark = [&](int i) -> hipError_t {
    return a.marks ? hipEventRecord((hipEvent_t)a.marks[i], st) : hipSuccess;
  };
  auto intra = [&](int wave, int64_t chunks, hipStream_t s) {
    if (a.T <= 0 || chunks <= 0) return;
    auto k = a.gate_mode == 2   ? intra_kernel<IO, D, C, 2>
             : a.gate_mode == 1 ? intra_kernel<IO, D, C, 1>
                                : intra_kernel<IO, D, C, 0>;
    hipLaunchKernelGGL(k, dim3((unsigned)(chunks * a.H)), dim3(NT_INTRA), 0, s, (const IO*)a.q,
                       (const IO*)a.k, (const IO*)a.v, a.g, a.beta, a.H, a.scale, table, recs,
                       a.A_log, a.dt_bias, a.lower_bound,
                       a.qk_heads > 0 ? a.qk_heads : a.H, a.per_head_gate, a.qk_l2norm,
                       (int)ws.ncb, wave_off, wave);
  };
  // a state launch over `nu_max` units of `units` (count *n_units) and, in
  // the first launch of a cut chain, the map units
  auto state = [&](const Unit* units, const int* n_units, int nu_max, const Unit* mu,
                   int nm_max) {
    const int64_t blocks = (int64_t)(a.H * nu_max + 7) / 8 * 8 * NV +
                           (int64_t)(a.H * nm_max + 7) / 8 * 8 * 2 * NV;
    hipLaunchKernelGGL((state_kernel<IO, D, C, VT>), dim3((unsigned)blocks), dim3(NTHREADS), 0,
                       st, seqs, units, n_units, nu_max, mu, counts + 1, recs, (int)ws.ncb, a.H,
                       a.h0, a.ht, (IO*)a.o, a.snaps, a.snap_rows, a.snap_interval, starts, maps);
  };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(NTHREADS), 0, st, a.cu_seqlens, a.N, a.T, C,
                     ws.ncb, a.snaps != nullptr ? a.snap_interval : 0, cut.seg_len,
                     cut.maps ? 1 : 0, cut.n_waves, table, seqs, units_a, units_m, units_c,
                     units_w, counts, wave_off);
  if ((e = mark(1)) != hipSuccess) return e;
  if (cut.n_waves > 1) {
    // waves: at most N segments of seg_len chunks each per wave
    const int64_t wave_chunks = std::min<int64_t>(ws.ncb, (int64_t)a.N * cut.seg_len);
    hipStream_t aux = nullptr;
    std::vector<hipEvent_t> ev;
    const bool two = !a.single_stream && stream_on_current_device(st) &&
                     !stream_capturing(st) &&
                     aux_acquire(cut.n_waves + 1, aux, ev) == hipSuccess;
    if (two) {
      // wave p's intra-chunk work on the second stream, its state pass on
      // the caller's stream once that is done
      if ((e = hipEventRecord(ev[cut.n_waves], st)) == hipSuccess &&
          (e = hipStreamWaitEvent(aux, ev[cut.n_waves], 0)) == hipSuccess) {
        for (int p = 0; p < cut.n_waves && e == hipSuccess; ++p) {
          intra(p, wave_chunks, aux);
          e = hipEventRecord(ev[p], aux);
        }
        if (e == hipSuccess && (e = mark(2)) == hipSuccess) {
          for (int p = 0; p < cut.n_waves && e == hipSuccess; ++p) {
            if ((e = hipStreamWaitEvent(st, ev[p], 0)) == hipSuccess)
              state(units_w + (size_t)p * a.N, counts + 0, a.N, nullptr, 0);
          }
        }
      }
      aux_release(ev);
      if (e != hipSuccess) return e;
    } else {
      for (int p = 0; p < cut.n_waves; ++p) intra(p, wave_chunks, st);
      if ((e = mark(2)) != hipSuccess) return e;
      for (int p = 0; p < cut.n_waves; ++p)
        state(units_w + (size_t)p * a.N, counts + 0, a.N, nullptr, 0);
    }
  } else {
    intra(0, ws.ncb, st);
    if ((e = mark(2)) != hipSuccess) return e;
    // first segments (every sequence, longest first) and, with maps, the
    // middle segments' maps in the same launch
    state(units_a, counts + 0, a.N, cut.maps ? units_m : nullptr, cut.maps ? (int)ws.nseg : 0);
    if (cut.maps) {
      // chain the start states, then re-run the later segments from them
      hipLaunchKernelGGL((scan_kernel<D>), dim3((unsigned)(a.N * a.H * (D / 4))), dim3(D), 0, st,
                         seqs, a.N, a.H, C, cut.seg_len, maps, starts);
      state(units_c, counts + 2, (int)ws.nseg, nullptr, 0);
    }
  }
  if ((e = mark(3)) != hipSuccess) return e;
  return hipGetLastError();
}

template <typename IO, int D>
hipError_t prefill_c(const PrefillArgs& a, hipStream_t st) {
  switch (a.C) {
    case 16: return launch_prefill<IO, D, 16>(a, st);
    case 32: return launch_prefill<IO, D, 32>(a, st);
    case 64: return launch_prefill<IO, D, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t prefill_d(const PrefillArgs& a, hipStream_t st) {
  switch (a.K) {
    case 16: return prefill_c<IO, 16>(a, st);
    case 32: return prefill_c<IO, 32>(a, st);
    case 64: return prefill_c<IO, 64>(a, st);
    case 128: return prefill_c<IO, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_workspace_bytes(int64_t T, int N, int H, int K, int V, int C) {
  (void)V;
  return ws_layout(T, N, H, K, C, rec_bytes(K, C)).total;
}

void prefill_schedule(int64_t T, int N, int H, int K, int C, int out[6]) {
  const StateCut cut = state_cut(T, N, H, K, C);
  const bool any = T > 0;
  out[0] = cut.n_waves;
  out[1] = cut.seg_len;
  out[2] = cut.maps ? 1 : 0;
  out[3] = any ? cut.n_waves : 0;
  out[4] = cut.maps ? 2 : cut.n_waves;
  out[5] = cut.maps ? 2 : 1;
}

hipError_t run_prefill(const PrefillArgs& a, hipStream_t stream) {
  return a.bf16_io ? prefill_d<bf16>(a, stream) : prefill_d<float>(a, stream);
}

}  // namespace kda
