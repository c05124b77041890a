// decode_args.h -- the persistent decode kernel's launch arguments, shared by the C ABI
// (which fills them from the caller's pointers) and the kernel.  Private to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfssm {
namespace decode {

struct Args {
    const uint8_t* in_bits;  // [L][8512][256]
    const float* in_sw;      // [L][8512]
    const int8_t* in_wa;     // [L][8512][16]
    const float* in_sa;      // [L][8512]
    const int8_t* in_wb;     // [L][16][2048]
    const float* in_sb;      // [L][16]
    const float* conv_w;     // [L][4352][4]
    const float* conv_b;     // [L][4352]
    const float* dt_bias;    // [L][64]
    const float* A_log;      // [L][64]
    const float* Dp;         // [L][64]
    const float* norm_w;     // [L][4096]
    const uint8_t* out_bits; // [L][2048][512]
    const float* out_sw;     // [L][2048]
    const int8_t* out_wa;    // [L][2048][16]
    const float* out_sa;     // [L][2048]
    const int8_t* out_wb;    // [L][16][4096]
    const float* out_sb;     // [L][16]
    const float* conv_in;    // [L][4352][4]
    float* conv_out;         // [L][4352][4]
    float* ssm_state;        // [L][64][64][128]
    const float* x_in;       // [2048]
    float* x_out;            // [2048]
    uint32_t* trace;         // optional [L][kTrWords]
    uint32_t* ws;            // workspace, kWsWords words
    int32_t* status;
    int L;
    float eps;
    int64_t spin_limit;
    uint32_t target_bias;    // 0; a test aid makes every wait unreachable with 1 << 30
};

}  // namespace decode

hipError_t launch_decode_layers(const decode::Args& a, hipStream_t stream);

}  // namespace dfssm
