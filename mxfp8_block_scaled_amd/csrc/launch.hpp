// Internal launchers behind the C ABI (one per kernel family).  Each assumes
// its arguments were validated by api.cpp and returns 0 or -7 (launch error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mxfp8 {

// Devices the per-device caches of the library cover (device ids 0..63).
constexpr int kMaxDevices = 64;

// Raises the dynamic LDS limit of kernel fn to `bytes` on the current device,
// once per device (the attribute belongs to a device's copy of the kernel):
// flags[dev] is 0 before, 1 after a successful call, 2 after a failed one.
// Returns false if the device is out of range or the runtime refused.
bool set_lds_limit_once(const void* fn, int bytes, std::atomic<int>* flags);

// MXFP8_OK if the current device is a gfx950 (cached per device).
int check_device_current();

// The host-side argument checks of mxfp8_linear (everything but the
// workspace and the device), and its launches once they passed (M >= 1,
// workspace of mxfp8_linear_workspace_bytes, device checked).
int linear_check_args(const void* x, int64_t M, int64_t K, int64_t ldx, const void* wp, const void* sp, int64_t N,
                      const void* bias, const void* y, int64_t ldy);
// cap: the workspace bytes the caller can give (SIZE_MAX: whatever the
// planned path needs); a planned slab path whose partials exceed it runs the
// decode or mid-M kernel, or the tile GEMM, instead.  linear_workspace_within
// is the workspace of the path so chosen.
size_t linear_workspace_within(int64_t M, int64_t N, int64_t K, size_t cap);
int linear_launch(const void* x, int64_t M, int64_t K, int64_t ldx, const void* wp, const void* sp, int64_t N,
                  const void* bias, void* y, int64_t ldy, void* workspace, hipStream_t stream, size_t cap);

int launch_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq, void* s,
                        int64_t lds, hipStream_t stream);

// Same, written as packed operand tiles (common.hpp), rows padded to 128.
int launch_quantize_act_packed(const void* x, int64_t M, int64_t K, int64_t ldx, void* qp, void* sp,
                               hipStream_t stream);

int launch_pack_weight(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws,
                       void* wp, void* sp, hipStream_t stream);

// Packs E stacked fused gate/up expert weights [E * 2I, K] with the row order
// of the MoE gate/up GEMM (moe.hip): within each expert, packed row
// p = 256 t + 128 h + q holds gate row 128 t + 64 h + q (q < 64) or up row
// I + 128 t + 64 h + q - 64 (q >= 64).  Requires I % 128 == 0.
int launch_pack_weight_gate_up(const void* w, const void* ws, int64_t E, int64_t I, int64_t K, void* wp, void* sp,
                               hipStream_t stream);

int launch_unpack_weight(const void* wp, const void* sp, int64_t N, int64_t K, void* w, void* ws,
                         hipStream_t stream);

// Large-tile GEMM on packed activations (qp, sp: M rows) and the packed
// weight (wp, wsp: N rows).  splits > 1 splits K across that many
// workgroups per tile: fp32 partials go to part (splits * M * round_up(N, 4)
// floats), then one reduce kernel adds them with the bias into y.
constexpr int kMaxSplitK = 8;
int device_cu_count();
int gemm_tile_splits(int64_t M, int64_t N, int64_t K);
int launch_gemm_tile(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp,
                     int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, int splits = 1,
                     void* part = nullptr);
// The same persistent tile GEMM with the weight as packed MXFP4 (W4A8, no
// K split; pack_weight_fp4's layout, scales as for MXFP8).
int launch_gemm_tile_w4(const void* qp, const void* sp, int64_t M, int64_t K, const void* w4p, const void* wsp,
                        int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream);

// y [M, N] (bf16, row stride ldy) = the sum of `splits` fp32 partials
// part[s][M][ldp] in split order, plus the bias, rounded once.
int launch_splitk_reduce(const float* part, int splits, int64_t M, int64_t N, int64_t ldp, const void* bias,
                         void* y, int64_t ldy, hipStream_t stream);

// Medium-tile GEMM on packed activations: one 128-row weight group x mt
// (128 or 64) activation rows per workgroup over the whole K (gemm_med.hip).
int launch_gemm_med(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp, int64_t N,
                    const void* bias, void* y, int64_t ldy, hipStream_t stream, int mt);

// Split-K slab GEMM (M <= kMidMaxM, any K) with the activation
// quantization fused in (gemm_slab.hip): each workgroup multiplies one
// 128-row weight group by one K slice of 2 * slab_steps_per_wave 128-K steps
// and writes an fp32 partial into ws (slab_ws_bytes); launch_splitk_reduce
// then adds the slices.
int slab_steps_per_wave(int64_t N, int64_t K);
size_t slab_ws_bytes(int64_t M, int64_t N, int64_t K);
int launch_gemm_slab(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                     const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws);
// The same with a packed MXFP4 weight (launch_pack_weight_fp4).
int launch_gemm_slab_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                         int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws);

// Skinny GEMM (M <= kSkinnyMaxM, K <= kSkinnyMaxK) with the activation
// quantization fused in; it needs no workspace (skinny_ws_bytes is the
// minimum the entry points ask for).
constexpr int64_t kSkinnyMaxM = 16;
constexpr int64_t kSkinnyMaxK = 8192;
inline size_t skinny_ws_bytes(int64_t, int64_t) { return 256; }

// Mid-M GEMM (kSkinnyMaxM < M <= kMidMaxM, K <= kSkinnyMaxK): the packed
// quantizer writes one 128-row group of activation tiles (E4M3 128 * K bytes,
// then the scale tiles, 128 * K / 32) into ws (mid_ws_bytes), then
// gemm_mid.hip's kernel reads them with the packed weight.
constexpr int64_t kMidMaxM = 128;
inline size_t mid_ws_bytes(int64_t, int64_t K) { return (size_t)(128 * K + 128 * (K / 32) + 255) / 256 * 256; }
int launch_gemm_mid(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp, int64_t N,
                    const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws);
// The same with a packed MXFP4 weight (launch_pack_weight_fp4).
int launch_gemm_mid_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                        int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws);
int launch_gemm_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                       int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws);
// The same with a packed MXFP4 weight (launch_pack_weight_fp4).
int launch_gemm_skinny_fp4(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                           int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream, void* ws);

// MXFP4 weights: w [N, K/2] bytes (two E2M1 per byte, element 2j in the low
// nibble; row stride ldw bytes), ws [N, K/32] UE8M0 -> packed tiles (pack.hip).
int launch_pack_weight_fp4(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws,
                           void* wp, void* sp, hipStream_t stream);
// Inverse: packed tiles -> w [N_pad, K/2] and ws [N_pad, K/32], contiguous.
int launch_unpack_weight_fp4(const void* wp, const void* sp, int64_t N, int64_t K, void* w, void* ws,
                             hipStream_t stream);
// Packed MXFP4 weight tiles -> packed MXFP8 tiles of the same values (the
// scales stay as they are), N_pad * K bytes.
int launch_widen_fp4(const void* w4, int64_t N, int64_t K, void* w8, hipStream_t stream);
// bf16 [M, K] -> MXFP4: E2M1 [M, K/2] (row stride ldq bytes) + UE8M0 [M, K/32].
int launch_quantize_fp4(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq, void* s,
                        int64_t lds, hipStream_t stream);

// Mixture of experts (moe.hip).
constexpr int64_t kGroupRowsHost = 128;   // = kGroupRows of common.hpp
constexpr int64_t kMoeMaxExperts = 256;
constexpr int64_t kMoeMaxTopk = 16;

// Device scratch of one MoE call, carved out of the caller's workspace.
struct MoeWorkspace {
  int* ids;          // [T*k] expert of row t*k + j
  float* wts;        // [T*k] routing weight
  int* blk_cnt;      // [nblk][E] rows of each route block per expert
  int* blk_off;      // [nblk][E] their offsets inside the expert's segment
  int* seg_off;      // [E] first sorted position of each expert
  int* meta;         // [0] M-tiles, [1] 128-row groups in use
  int* tile_e;       // [mt_max] expert of each M-tile
  int* tile_g0;      // [mt_max] its first 128-row group
  int* tile_ng;      // [mt_max] its groups (1 or 2)
  int* sorted_row;   // [p_max] row t*k + j at each sorted position, -1 = pad
  uint8_t* xq;       // MXFP8 token rows, row-major [T + 1, H] (row T all zero)
  uint8_t* xs;       // their scales [T + 1, H / 32]
  uint8_t* a1s;      // packed scales of the expert-sorted token rows [p_max, H / 32]
  uint8_t* a2q;      // packed MXFP8 gated activations [p_max, I]
  uint8_t* a2s;
  float* ys;         // expert output rows, fp32 [T*k + 1, H], row t*k + j (row T*k: spare)
  int64_t p_max;     // sorted positions (multiple of 128, one spare group)
  int64_t mt_max;    // upper bound of M-tiles
};

struct MoeArgs {
  const void* x;       // bf16 [T, H]
  const float* logits; // fp32 [T, E]
  int64_t T, H, E, topk, I;
  const void* w13p;
  const void* s13p;
  const void* w2p;
  const void* s2p;
  void* y;             // bf16 [T, H]
  void* dbg_act;       // optional bf16 [T*k, I]
  void* dbg_q;         // optional E4M3 [T*k, I]
  void* dbg_s;         // optional UE8M0 [T*k, I/32]
  void* dbg_ids;       // optional int32 [T*k] routed expert
  void* dbg_wts;       // optional fp32 [T*k] routing weight
  MoeWorkspace ws;
};

int launch_moe(const MoeArgs& a, hipStream_t stream);

}  // namespace mxfp8
