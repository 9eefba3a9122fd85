// Internal interfaces between the C-ABI host layer (abi.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mlb {

struct AppendArgs {
  const uint16_t* latent;
  const uint16_t* k_rope;
  const int64_t* slot_mapping;
  const int32_t* seq_slot;
  const int32_t* pos;
  const int32_t* new_len;
  int32_t T;
  uint8_t* pages;
  int64_t num_pages;
  uint16_t* prot;
  int32_t num_seq_slots;
};

struct DecodeArgs {
  const uint16_t* q_lat;
  const uint16_t* q_rope;
  const uint8_t* pages;
  int64_t num_pages;
  const uint16_t* prot;
  int32_t num_seq_slots;
  const int32_t* seq_slot;
  const int32_t* block_table;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t max_seq_len;   // host bound, already min(max_seq_len, max_blocks*64)
  int32_t B, H;          // H: query rows per sequence (nq queries x hq heads)
  int32_t nq, hq;        // queries per sequence and heads per query: row r is
                         // query r / hq, which sees the first L - (nq-1-r/hq) tokens
  float scale_log2;      // softmax_scale * log2(e)
  int32_t pps;           // pages per split
  int32_t nsplit;        // splits of a max_seq_len sequence (grid.x)
  int32_t balance;       // deal the B * nsplit slots by sequence length (split_map.h)
  float* ws_o;           // [B][nsplit][H][512] unnormalised partial outputs
  float* ws_ml;          // [B][nsplit][H][4]   (max in log2 units, bf16-weight sum, fp32 sum, 0)
  float* out;            // [B][H][512]
  float* lse;            // [B][H]
  // fused writer (null new_c: decode only): token seq_lens[b]-1 of sequence
  // b is new_c[b] / new_r[b]; the kernel stores its packed copy and bf16
  // protection row, and reads that token from new_c / new_r
  const uint16_t* new_c;  // [B][512] bf16
  const uint16_t* new_r;  // [B][64]  bf16
  uint8_t* wpages;        // == pages
  uint16_t* wprot;        // == prot
};

// Which decode kernel serves `rows` query rows per sequence (a multiple of
// 16): the 16-row kernel reconstructs each page once per 16 rows, the 128-row
// kernel once per block of up to 128 rows (rows past the last multiple of 128
// are padding it masks).  Measured on MI355X at batch 32 x 8192 C4R4 tokens, a
// 128-row block costs about as much as five 16-row groups (64 rows: 0.109 ms
// with 16-row groups, 0.149 ms padded; 96 rows: 0.187 vs 0.155 ms), so the
// 128-row kernel is taken when 5 * ceil(rows / 128) < ceil(rows / 16).
inline bool use_rows128(int32_t rows) {
  const int64_t r = rows;
  return 5 * ((r + 127) / 128) < (r + 15) / 16;
}

// Split plan: how a max_seq_len sequence is cut into splits.
struct Plan {
  int32_t pps;       // pages per split (>= 1)
  int32_t nsplit;    // number of splits of a max-length sequence (>= 1)
  size_t ws_bytes;   // workspace needed (0 when nsplit == 1)
  bool too_large;    // the workspace would pass 2^60 bytes: the call is refused
};

// ws_cap > 0: the automatic plan (num_splits == 0) takes no more splits than
// a workspace of ws_cap bytes holds (a single split when not even two fit).
Plan make_plan(int32_t B, int32_t H, int32_t max_seq_len, int32_t num_splits,
               size_t ws_cap = 0);

// Host-side validation and plan of a decode call (no HIP call), and the
// workspace pointers of the plan; both in abi.cpp.
int decode_setup(int f, const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* pages,
                 int64_t num_pages, const uint16_t* prot, int32_t num_seq_slots,
                 const int32_t* seq_slot, const int32_t* block_table, int32_t max_blocks,
                 const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t H,
                 float softmax_scale, int32_t num_splits, float* out, float* lse,
                 const uint16_t* new_c, const uint16_t* new_r, int32_t nq, size_t ws_cap,
                 DecodeArgs& a, Plan& plan);
void set_workspace(DecodeArgs& a, const Plan& plan, void* workspace);

int launch_append(int f, const AppendArgs& a, hipStream_t stream);
int launch_decode(int f, const DecodeArgs& a, hipStream_t stream);
int launch_decode128(int f, const DecodeArgs& a, hipStream_t stream);   // H % 128 == 0
int launch_decode16w(int f, const DecodeArgs& a, hipStream_t stream);   // other H
int launch_dequant_dump(int f, const uint8_t* pages, int64_t page_id, uint16_t* out,
                        hipStream_t stream);

}  // namespace mlb
