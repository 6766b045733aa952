// Decode attention over a rank's local heads (one query token per sequence).
//
// At decode the key/value cache is the dominant byte stream.  With grouped KV
// heads, the G = Hq/Hkv query heads of one KV head read the same cached keys
// and values, so one workgroup serves all G heads of one (sequence, KV head)
// pair over a chunk of the key span and every cached byte is read once.  The
// span is split into chunks so that about one workgroup per CU runs
// (flash-decoding split-KV); each chunk writes an unnormalised partial (max,
// sum of exponentials, weighted value sum) and a second pass combines the
// chunks with log-sum-exp rescaling, in chunk order.
//
// The G heads are the query columns of a small attention problem: S^T = K Q^T
// on v_mfma_f32_32x32x16_bf16 with the heads padded to 32 columns (the MFMA
// work is far below the chip's rate at these byte counts), so a lane owns one
// head and 16 of a tile's 32 keys, and the softmax statistics are an
// in-register reduction plus one v_permlane32_swap.  The probabilities feed
// O^T = V^T P^T directly, with V^T read from V ([key][d] in LDS) by
// ds_read_b64_tr_b16 (the layouts of the prefill kernel).
//
// Each of the 4 waves streams its own contiguous run of 32-key tiles through
// a private two-stage LDS ring with buffer_load_dwordx4 ... lds (1 KB = 4 key
// rows per load, rows past the span reading as zero, non-temporal since each
// cached byte is read once per step): the next tile's K and V
// are in flight while the current one is computed, with an online softmax
// across tiles.  There is no barrier in the loop; the waves' (max, sum, O^T)
// are merged through LDS at the end.
//
// Paged variant (page P1 "Tensor parallel 对 KV cache 的影响": the block table
// is the same on every rank, each rank's physical blocks hold only its own KV
// heads): key t of sequence b sits in physical block table[b][t / bs], slot
// t % bs, of the rank's K and V pools.  A workgroup first copies the table
// entries of its key chunk to LDS; each 1 KB load (4 key rows) then lies in one
// block (bs is a multiple of 16), so its buffer resource is based at that
// block and bounded to it.  Sequences have their own lengths; entries outside
// [0, num_blocks) read as zero instead of faulting.
//
// Fused append (kn != nullptr): the decode step's own k and v rows are stored
// to their cache slot by the first wave of chunk 0 (contiguous: position
// Skv - 1; paged: context_lens[b] - 1, skipped where the append would skip
// it), and the wave whose tile holds key L - 1 writes those rows over the
// cached ones in its landed LDS tile before reading it.  The result equals
// the append launch followed by the attention launch, bit for bit, without
// the attention depending on the store.
#include <algorithm>

#include <mutex>

#include "common.h"

namespace tpl {

constexpr int kDecD = 128;           // head dimension handled
constexpr int kDecTile = 32;         // keys per tile
constexpr int kDecMaxG = 32;         // query heads per KV head (MFMA columns)

constexpr int kPagedMaxBlocks = 512;   // table entries one workgroup stages in LDS

struct DecArgs {
  const uint16_t* q; int64_t qs0, qs2;          // (b, h) strides (s = 0)
  // contiguous: element (b, t, j, d) at k[b*ks0 + t*ks1 + j*ks2 + d];
  // paged:      element (block, slot, j, d) at k[block*ks0 + slot*ks1 + j*ks2 + d]
  const uint16_t* k; const uint16_t* v; int64_t ks0, ks1, ks2;
  uint16_t* o; int64_t os0, os2;
  float* ws;                                    // partials, or nullptr if one chunk
  int Skv, Hq, Hkv, G, nsplit, chunk;           // chunk: keys per workgroup (multiple of 4*32)
  float scale_log2;                             // softmax scale * log2(e)
  // paged only
  const int* table; int64_t tstride; const int* lens; int bs; int64_t nblocks;
  // fused append only (else kn == nullptr): element (b, j, d) of the new rows at
  // kn[b*nstride + j*D + d]; kst, vst: the caches (pools) written
  const uint16_t* kn; const uint16_t* vn; int64_t nstride;
  uint16_t* kst; uint16_t* vst;
};

namespace {
typedef short dec_s16x4 __attribute__((ext_vector_type(4)));
#define TPL_DLDS __attribute__((address_space(3)))

__device__ __forceinline__ float dec_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float dec_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace

template <bool PAGED>
__global__ __launch_bounds__(256) void attn_decode_kernel(DecArgs a) {
  constexpr int TE = kDecTile * kDecD;                 // bf16 elements of one K (or V) tile
  constexpr int WRING = 2 * 2 * TE;                    // per wave: 2 stages x (K, V)
  // One LDS object: the rings (128 KB), then the waves' softmax statistics
  // (1 KB) and the paged variant's copy of the chunk's table entries (2 KB).
  // With a second __shared__ object the compiler can no longer tell the ring
  // reads from the in-flight direct-to-LDS writes and waits for all of them
  // before each tile's reads, which defeats the two-stage ring.
  constexpr int STAT_E = 4 * kDecMaxG * 2 * 2;          // bf16-sized elements of wstat
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * WRING + STAT_E + (PAGED ? 2 * kPagedMaxBlocks : 0)];
  auto wstat = reinterpret_cast<float (*)[kDecMaxG][2]>(lds + 4 * WRING);
  int* tbl = reinterpret_cast<int*>(lds + 4 * WRING + STAT_E);

  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hl = lane >> 5;
  const int G = a.G;
  // keys of this sequence (paged: its own length, clamped into [1, Skv])
  const int L = PAGED ? min(max(a.lens[b], 1), a.Skv) : a.Skv;
  const int wkeys = a.chunk / 4;                       // keys per wave (multiple of 32)
  const int tw = split * a.chunk + wave * wkeys;       // first key of this wave
  const int nt = max(0, min(wkeys, L - tw) + kDecTile - 1) / kDecTile;   // tiles with keys

  // Fused append: where this sequence's new rows go (pos_new, slot offset dst)
  // and whether they stand in for key L - 1 of the attention.  All uniform.
  bool store_ok = false, subst = false;
  int64_t dst = 0;
  if (a.kn != nullptr) {
    if constexpr (PAGED) {
      const int pos_new = a.lens[b] - 1;
      int pb = -1;
      if (pos_new >= 0 && pos_new / a.bs < a.tstride) pb = a.table[(int64_t)b * a.tstride + pos_new / a.bs];
      store_ok = pb >= 0 && pb < a.nblocks;
      dst = (int64_t)pb * a.ks0 + (int64_t)(pos_new % a.bs) * a.ks1 + (int64_t)j * a.ks2;
      subst = store_ok && pos_new == L - 1;
    } else {
      store_ok = subst = true;
      dst = (int64_t)b * a.ks0 + (int64_t)(L - 1) * a.ks1 + (int64_t)j * a.ks2;
    }
  }
  const bool wave_store = store_ok && split == 0 && wave == 0;
  const bool wave_subst = subst && L - 1 >= tw && L - 1 < tw + wkeys;
  uint32_t knew = 0u, vnew = 0u;   // d = 2 lane, 2 lane + 1 of the new rows
  if (wave_store || wave_subst) {
    const int64_t src = (int64_t)b * a.nstride + (int64_t)j * kDecD + 2 * lane;
    knew = *reinterpret_cast<const uint32_t*>(a.kn + src);
    vnew = *reinterpret_cast<const uint32_t*>(a.vn + src);
  }
  if (wave_store) {
    *reinterpret_cast<uint32_t*>(a.kst + dst + 2 * lane) = knew;
    *reinterpret_cast<uint32_t*>(a.vst + dst + 2 * lane) = vnew;
  }
  const int tnew = wave_subst ? (L - 1 - tw) / kDecTile : -1;   // tile of this wave holding it

  const int blk0 = PAGED ? split * a.chunk / a.bs : 0;   // first table entry of the chunk
  if constexpr (PAGED) {
    const int nb = min((split * a.chunk + a.chunk - 1) / a.bs, (L - 1) / a.bs) - blk0 + 1;
    for (int e = tid; e < nb; e += 256) tbl[e] = a.table[(int64_t)b * a.tstride + blk0 + e];
    __syncthreads();
  }

  const uint32_t nrec = PAGED ? (uint32_t)(((int64_t)(a.bs - 1) * a.ks1 + kDecD) * 2)
                              : (uint32_t)(((int64_t)(L - 1) * a.ks1 + kDecD) * 2);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + b * a.ks0 + j * a.ks2), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v + b * a.ks0 + j * a.ks2), 0, nrec, 0x00020000);
  TPL_DLDS uint16_t* ring = (TPL_DLDS uint16_t*)lds + wave * WRING;
  const int lr = lane >> 4, lp = lane & 15;
  // tile i of this wave -> stage i & 1: 8 loads of 4 rows for K, 8 for V
  auto issue = [&](int i) {
    TPL_DLDS uint16_t* kd = ring + (i & 1) * 2 * TE;
    TPL_DLDS uint16_t* vd = kd + TE;
    // Paged: the tile starts at a multiple of 32 keys and bs is a multiple of
    // 16, so each 16-row half of the tile lies in one block: two table
    // lookups and four buffer resources per tile.  A half that starts past
    // the span, or whose entry is outside [0, nblocks), gets an empty
    // resource (zeros); rows past the span inside a valid half read zero
    // through their per-lane offsets.
    __amdgpu_buffer_rsrc_t pk[2], pv[2];
    if constexpr (PAGED) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int t0 = tw + i * kDecTile + 16 * hf;
        int pb = (t0 < L && i < nt) ? tbl[t0 / a.bs - blk0] : -1;
        pb = __builtin_amdgcn_readfirstlane(pb);
        const bool bok = pb >= 0 && pb < a.nblocks;
        const int64_t base = (bok ? pb * a.ks0 : 0) + j * a.ks2;
        pk[hf] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + base), 0, bok ? nrec : 0u, 0x00020000);
        pv[hf] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + base), 0, bok ? nrec : 0u, 0x00020000);
      }
    }
#pragma unroll
    for (int u = 0; u < kDecTile / 4; ++u) {
      const int row = 4 * u + lr;
      const int t = tw + i * kDecTile + row;
      const bool ok = t < L && i < nt;
      const int kc = lp ^ (row & 15), vc = lp ^ (4 * (row & 3));
      if constexpr (PAGED) {
        const uint32_t rb = (uint32_t)((int64_t)(t % a.bs) * a.ks1 * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pk[u >= 4], (TPL_DLDS void*)(kd + u * 4 * kDecD), 16,
                                                 ok ? rb + (uint32_t)kc * 16u : 0x80000000u, 0, 0, kLoadStream);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pv[u >= 4], (TPL_DLDS void*)(vd + u * 4 * kDecD), 16,
                                                 ok ? rb + (uint32_t)vc * 16u : 0x80000000u, 0, 0, kLoadStream);
      } else {
        const uint32_t rb = (uint32_t)((int64_t)t * a.ks1 * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (TPL_DLDS void*)(kd + u * 4 * kDecD), 16,
                                                 ok ? rb + (uint32_t)kc * 16u : 0x80000000u, 0, 0, kLoadStream);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (TPL_DLDS void*)(vd + u * 4 * kDecD), 16,
                                                 ok ? rb + (uint32_t)vc * 16u : 0x80000000u, 0, 0, kLoadStream);
      }
    }
  };
  issue(0);

  // Q^T fragments: column c32 = query head j*G + c32 (zero past G), d = 16 kk + 8 hl .. +7
  bf16x8 qf[8];
  {
    const bool hv = c32 < G;
    const uint16_t* qrow = a.q + b * a.qs0 + (int64_t)(j * G + (hv ? c32 : 0)) * a.qs2;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v4 = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hl * 8);
      if (!hv) v4 = u32x4{0u, 0u, 0u, 0u};
      qf[kk] = as_bf16x8(v4);
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const int g16 = lane >> 4, sidx = lane & 15;
  const int tr_row = sidx >> 2, tr_d = 16 * (g16 & 1) + 4 * (sidx & 3);

  for (int i = 0; i < nt; ++i) {
    // the other stage was last read by tile i-1, whose reads completed before its MFMAs
    issue(i + 1);
    __builtin_amdgcn_s_waitcnt((16 & 15) | ((16 >> 4) << 14) | 0x0F70);   // tile i landed; tile i+1 (16 loads) may pend
    if (i == tnew) {   // fused append: the new rows replace the cached key L - 1
      uint16_t* kt = lds + wave * WRING + (i & 1) * 2 * TE;
      const int r = L - 1 - (tw + i * kDecTile);
      const int c = lane >> 2, e = 2 * (lane & 3);   // 16-byte chunk and element of d = 2 lane
      *reinterpret_cast<uint32_t*>(kt + r * kDecD + (c ^ (r & 15)) * 8 + e) = knew;
      *reinterpret_cast<uint32_t*>(kt + TE + r * kDecD + (c ^ (4 * (r & 3))) * 8 + e) = vnew;
    }
    const uint16_t* ks = lds + wave * WRING + (i & 1) * 2 * TE;
    const uint16_t* vs = ks + TE;
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int ch = (2 * kk + hl) ^ (c32 & 15);
      const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + c32 * kDecD + ch * 8));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], st, 0, 0, 0);
    }
    // online softmax for column c32 over this tile's 32 keys (16 here, 16 in lane ^ 32)
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] *= a.scale_log2;
    const int t0 = tw + i * kDecTile;
    if (t0 + kDecTile > L) {   // wave-uniform: only the span's last tile is ragged
      // key t0 + 4 hl + 8 (r / 4) + r % 4 is valid while it is < L
      const int rel = L - (t0 + 4 * hl);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= rel) st[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[r]);
    mx = dec_pair_max(mx);
    const float mnew = fmaxf(mrun, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    // v_exp_f32 directly: arguments are <= 0 and results below 2^-126 may flush to zero
    const float alpha = __builtin_amdgcn_exp2f(mrun - muse);
    mrun = mnew;
    bf16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(st[half * 8 + e] - muse);
        psum += p[e];
      }
      pb[half] = as_bf16x8(pack8(p));
    }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    // O^T[d, col] += V^T[d, keys] P^T[keys, col]; step `half` covers keys
    // 16 half + {4 hl + 0..3, 8 + 4 hl + 0..3} (the P^T register order).
    // The V^T fragments come from 16 transposing reads (row r0 and r0 + 8,
    // 2048 bytes further, share the chunk swizzle).  They are issued by one
    // asm block that also waits for them: the compiler would otherwise wait
    // for every load in flight, the next tile's included, before its own
    // ds_read_b64_tr_b16, because it cannot tell that they read the other
    // stage.
    u32x2 vf[2][4][2];
    {
      uint32_t va[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = 32 * db + tr_d, r0 = half * 16 + 4 * hl + tr_row;
          va[half][db] = (uint32_t)reinterpret_cast<uintptr_t>(
              (TPL_DLDS uint16_t*)vs + r0 * kDecD + ((d >> 3) ^ (4 * (r0 & 3))) * 8 + (d & 7));
        }
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %16 offset:2048\n\t"
          "ds_read_b64_tr_b16 %2, %17\n\tds_read_b64_tr_b16 %3, %17 offset:2048\n\t"
          "ds_read_b64_tr_b16 %4, %18\n\tds_read_b64_tr_b16 %5, %18 offset:2048\n\t"
          "ds_read_b64_tr_b16 %6, %19\n\tds_read_b64_tr_b16 %7, %19 offset:2048\n\t"
          "ds_read_b64_tr_b16 %8, %20\n\tds_read_b64_tr_b16 %9, %20 offset:2048\n\t"
          "ds_read_b64_tr_b16 %10, %21\n\tds_read_b64_tr_b16 %11, %21 offset:2048\n\t"
          "ds_read_b64_tr_b16 %12, %22\n\tds_read_b64_tr_b16 %13, %22 offset:2048\n\t"
          "ds_read_b64_tr_b16 %14, %23\n\tds_read_b64_tr_b16 %15, %23 offset:2048\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(vf[0][0][0]), "=&v"(vf[0][0][1]), "=&v"(vf[0][1][0]), "=&v"(vf[0][1][1]),
            "=&v"(vf[0][2][0]), "=&v"(vf[0][2][1]), "=&v"(vf[0][3][0]), "=&v"(vf[0][3][1]),
            "=&v"(vf[1][0][0]), "=&v"(vf[1][0][1]), "=&v"(vf[1][1][0]), "=&v"(vf[1][1][1]),
            "=&v"(vf[1][2][0]), "=&v"(vf[1][2][1]), "=&v"(vf[1][3][0]), "=&v"(vf[1][3][1])
          : "v"(va[0][0]), "v"(va[0][1]), "v"(va[0][2]), "v"(va[0][3]),
            "v"(va[1][0]), "v"(va[1][1]), "v"(va[1][2]), "v"(va[1][3])
          : "memory");
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 l2 = vf[half][db][0], h2 = vf[half][db][1];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]}),
                                                           pb[half], oacc[db], 0, 0, 0);
      }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // the trailing (out-of-range) DMA has landed
  const float lsum = dec_pair_sum(lrun);

  // merge the 4 waves: per column, O = sum_w 2^(m_w - m) O_w, L = sum_w 2^(m_w - m) l_w
  __syncthreads();   // every wave is done with its ring
  float* red = reinterpret_cast<float*>(lds);   // [4 waves][32 cols][128 d]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = db * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
      red[(wave * kDecMaxG + c32) * kDecD + d] = oacc[db][r];
    }
  if (hl == 0) { wstat[wave][c32][0] = mrun; wstat[wave][c32][1] = lsum; }
  __syncthreads();
  for (int e = tid; e < G * kDecD; e += 256) {
    const int c = e / kDecD, d = e % kDecD;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, wstat[w][c][0]);
    const float mu = (m == -INFINITY) ? 0.f : m;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = exp2f(wstat[w][c][0] - mu);
      num = fmaf(sc, red[(w * kDecMaxG + c) * kDecD + d], num);
      den = fmaf(sc, wstat[w][c][1], den);
    }
    const int h = j * G + c;
    if (a.ws == nullptr) {
      a.o[b * a.os0 + h * a.os2 + d] = (uint16_t)f2bf_bits(num / den);
    } else {
      // ws layout: [B][Hq][nsplit] x {m, l} followed by [B][Hq][nsplit][D]
      const int64_t row = ((int64_t)b * a.Hq + h) * a.nsplit + split;
      float* ml = a.ws;
      float* ov = a.ws + (int64_t)gridDim.z * a.Hq * a.nsplit * 2;
      ov[row * kDecD + d] = num;
      if (d == 0) { ml[row * 2] = m; ml[row * 2 + 1] = den; }
    }
  }
}

// Combine the chunk partials of one (sequence, head): 128 threads, one per
// output element, chunks visited in order.  Partials are loaded 8 chunks at a
// time (indices clamped into range and masked afterwards, so the loads carry
// no branches and are all in flight together).
__global__ __launch_bounds__(128) void attn_decode_combine_kernel(DecArgs a, int B) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* ml = a.ws;
  const float* ov = a.ws + (int64_t)B * a.Hq * a.nsplit * 2;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.nsplit;
  const int ns = a.nsplit;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float m[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = ml[(row0 + min(s0 + u, ns - 1)) * 2];
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmaxf(mx, m[u]);   // clamped duplicates do not change the max
  }
  float num = 0.f, den = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float m[8], l[8], o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t r = row0 + min(s0 + u, ns - 1);
      m[u] = ml[r * 2];
      l[u] = ml[r * 2 + 1];
      o[u] = ov[r * kDecD + d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool use = s0 + u < ns && l[u] != 0.f;   // past the end, or an empty chunk
      const float w = use ? exp2f(m[u] - mx) : 0.f;
      num = fmaf(w, use ? o[u] : 0.f, num);
      den = fmaf(w, use ? l[u] : 0.f, den);
    }
  }
  a.o[b * a.os0 + h * a.os2 + d] = (uint16_t)f2bf_bits(num / den);
}

// Chunks of whole 4 x 32-key tiles per workgroup, about one workgroup per CU
// (256) over all (sequence, KV head) pairs.
static int dec_chunk(int64_t B, int64_t Hkv, int64_t Skv) {
  const int64_t pairs = B * Hkv;
  int64_t ns = (256 + pairs - 1) / pairs;
  const int64_t max_ns = (Skv + 4 * kDecTile - 1) / (4 * kDecTile);
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  int64_t chunk = (Skv + ns - 1) / ns;
  chunk = (chunk + 4 * kDecTile - 1) / (4 * kDecTile) * (4 * kDecTile);
  return (int)chunk;
}

int attn_decode_nsplit(int64_t B, int64_t Hkv, int64_t Skv) {
  const int64_t chunk = dec_chunk(B, Hkv, Skv);
  return (int)((Skv + chunk - 1) / chunk);
}

size_t attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv) {
  const int ns = attn_decode_nsplit(B, Hkv, Skv);
  if (ns == 1) return 0;
  return (size_t)(B * Hq * ns) * (2 + kDecD) * sizeof(float);
}

tp_status attn_decode(const void* q, const int64_t qs[3], const void* k, const void* v,
                      const int64_t kvs[3], void* o, const int64_t os[3], int64_t B, int64_t Skv,
                      int64_t Hq, int64_t Hkv, float scale, void* ws, hipStream_t s,
                      const void* kn, const void* vn, int64_t nstride) {
  DecArgs a;
  a.kn = static_cast<const uint16_t*>(kn); a.vn = static_cast<const uint16_t*>(vn); a.nstride = nstride;
  a.kst = const_cast<uint16_t*>(static_cast<const uint16_t*>(k));
  a.vst = const_cast<uint16_t*>(static_cast<const uint16_t*>(v));
  a.q = static_cast<const uint16_t*>(q); a.qs0 = qs[0]; a.qs2 = qs[2];
  a.k = static_cast<const uint16_t*>(k); a.v = static_cast<const uint16_t*>(v);
  a.ks0 = kvs[0]; a.ks1 = kvs[1]; a.ks2 = kvs[2];
  a.o = static_cast<uint16_t*>(o); a.os0 = os[0]; a.os2 = os[2];
  a.Skv = (int)Skv; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv);
  if (a.G > kDecMaxG) return TP_ERR_UNSUPPORTED;
  a.chunk = dec_chunk(B, Hkv, Skv);
  a.nsplit = attn_decode_nsplit(B, Hkv, Skv);
  a.ws = a.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.table = nullptr; a.tstride = 0; a.lens = nullptr; a.bs = 0; a.nblocks = 0;
  hipLaunchKernelGGL(attn_decode_kernel<false>, dim3(a.nsplit, a.Hkv, B), dim3(256), 0, s, a);
  if (a.ws) hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.Hq, B), dim3(128), 0, s, a, (int)B);
  TPL_LAUNCH_CHECK("attn_decode");
  return TP_OK;
}

// Paged decode: chunks also bounded so that one chunk's table entries fit the
// workgroup's LDS copy.
static int paged_chunk(int64_t B, int64_t Hkv, int64_t max_len, int64_t bs) {
  int chunk = dec_chunk(B, Hkv, max_len);
  const int64_t cap = (int64_t)(kPagedMaxBlocks - 1) * bs / (4 * kDecTile) * (4 * kDecTile);
  if (chunk > cap) chunk = (int)cap;
  return chunk;
}

int attn_paged_nsplit(int64_t B, int64_t Hkv, int64_t max_len, int64_t bs) {
  const int64_t chunk = paged_chunk(B, Hkv, max_len, bs);
  return (int)((max_len + chunk - 1) / chunk);
}

size_t attn_paged_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_len, int64_t bs) {
  const int ns = attn_paged_nsplit(B, Hkv, max_len, bs);
  if (ns == 1) return 0;
  return (size_t)(B * Hq * ns) * (2 + kDecD) * sizeof(float);
}

tp_status attn_decode_paged(const void* q, const int64_t qs[2], const void* kp, const void* vp,
                            const int64_t ps[3], int64_t nblocks, const int* table, int64_t tstride,
                            const int* lens, int64_t max_len, int64_t bs, void* o,
                            const int64_t os[2], int64_t B, int64_t Hq, int64_t Hkv, float scale,
                            void* ws, hipStream_t s, const void* kn, const void* vn,
                            int64_t nstride) {
  DecArgs a;
  a.kn = static_cast<const uint16_t*>(kn); a.vn = static_cast<const uint16_t*>(vn); a.nstride = nstride;
  a.kst = const_cast<uint16_t*>(static_cast<const uint16_t*>(kp));
  a.vst = const_cast<uint16_t*>(static_cast<const uint16_t*>(vp));
  a.q = static_cast<const uint16_t*>(q); a.qs0 = qs[0]; a.qs2 = qs[1];
  a.k = static_cast<const uint16_t*>(kp); a.v = static_cast<const uint16_t*>(vp);
  a.ks0 = ps[0]; a.ks1 = ps[1]; a.ks2 = ps[2];
  a.o = static_cast<uint16_t*>(o); a.os0 = os[0]; a.os2 = os[1];
  a.Skv = (int)max_len; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv);
  if (a.G > kDecMaxG) return TP_ERR_UNSUPPORTED;
  a.chunk = paged_chunk(B, Hkv, max_len, bs);
  a.nsplit = attn_paged_nsplit(B, Hkv, max_len, bs);
  a.ws = a.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.table = table; a.tstride = tstride; a.lens = lens; a.bs = (int)bs; a.nblocks = nblocks;
  hipLaunchKernelGGL(attn_decode_kernel<true>, dim3(a.nsplit, a.Hkv, B), dim3(256), 0, s, a);
  if (a.ws) hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.Hq, B), dim3(128), 0, s, a, (int)B);
  TPL_LAUNCH_CHECK("attn_decode_paged");
  return TP_OK;
}

// ---- a library-owned partials buffer for callers that cannot allocate ----------

// attn_decode_workspace over every call the contiguous decode entry points
// accept is at most this: a call splits its key span only when it has at most
// 255 (sequence, KV head) pairs, into at most ceil(256 / pairs) chunks each,
// so B * Hkv * nsplit <= 510 and B * Hq * nsplit <= 32 * 510 partial rows of
// (2 + 128) floats (8,486,400 bytes).
constexpr size_t kDecScratchBytes = size_t(kDecMaxG) * 510 * (2 + kDecD) * sizeof(float);

// Every call of the allocation-free entry point on a GPU uses that GPU's copy
// of this array (held until the process ends).  The chunk partials are fully
// written by the attention kernel before the combine kernel reads them, so
// nothing in it needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kDecScratchBytes];

// Device address of `scratch` on the device of stream s (the current device
// for the null stream).  The address is looked up once per device, with that
// device current, and kept; host code never passes the array's name itself.
tp_status attn_decode_scratch(hipStream_t s, void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) { set_hip_error("hipGetDevice", e); return TP_ERR_HIP; }
  int dev = cur;
  if (s != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(s, &d);
    if (e != hipSuccess) { set_hip_error("hipStreamGetDevice", e); return TP_ERR_HIP; }
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return TP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) {
      set_hip_error("hipSetDevice", e);
      return TP_ERR_HIP;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || p == nullptr) {
      set_hip_error("hipGetSymbolAddress(scratch)", e != hipSuccess ? e : hipErrorInvalidSymbol);
      return TP_ERR_HIP;
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kDecScratchBytes;
  return TP_OK;
}

// Write the current token's k and v of every sequence into its slot
// (lens[b] - 1) of the paged pools; sequences whose slot or block is out of
// range are skipped.
__global__ __launch_bounds__(256) void paged_kv_append_kernel(
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, int64_t new_stride,
    uint16_t* __restrict__ kp, uint16_t* __restrict__ vp, int64_t ps0, int64_t ps1, int64_t ps2,
    int64_t nblocks, const int* __restrict__ table, int64_t tstride, int64_t maxblk,
    const int* __restrict__ lens, int64_t B, int64_t H, int64_t D, int64_t bs) {
  const int64_t total = B * H * D;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = e % D, j = (e / D) % H, b = e / (D * H);
    const int64_t pos = (int64_t)lens[b] - 1;
    if (pos < 0 || pos / bs >= maxblk) continue;
    const int64_t pb = table[b * tstride + pos / bs];
    if (pb < 0 || pb >= nblocks) continue;
    const int64_t src = b * new_stride + j * D + d;
    const int64_t dst = pb * ps0 + (pos % bs) * ps1 + j * ps2 + d;
    kp[dst] = kn[src];
    vp[dst] = vn[src];
  }
}

tp_status paged_kv_append(const void* kn, const void* vn, int64_t new_stride, void* kp, void* vp,
                          const int64_t ps[3], int64_t nblocks, const int* table, int64_t tstride,
                          int64_t maxblk, const int* lens, int64_t B, int64_t H, int64_t D, int64_t bs,
                          hipStream_t s) {
  const int64_t total = B * H * D;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(paged_kv_append_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const uint16_t*>(kn), static_cast<const uint16_t*>(vn), new_stride,
                     static_cast<uint16_t*>(kp), static_cast<uint16_t*>(vp), ps[0], ps[1], ps[2],
                     nblocks, table, tstride, maxblk, lens, B, H, D, bs);
  TPL_LAUNCH_CHECK("paged_kv_append");
  return TP_OK;
}

}  // namespace tpl
