// Kernel lookup: each (weight type, batch tile) instantiation unit
// (kernels.hip compiled with MK_WT / MK_NB) exports one accessor.
#pragma once

namespace mk {
enum KernelKind { KK_PERSISTENT = 0, KK_LEVEL_GEMV = 1, KK_LEVEL_ATTN = 2 };
}

extern "C" {
void* mk_kernels_bf16_1(int kind);
void* mk_kernels_bf16_1s(int kind);
void* mk_kernels_bf16_2(int kind);
void* mk_kernels_bf16_4(int kind);
void* mk_kernels_bf16_8(int kind);
void* mk_kernels_bf16_16(int kind);
void* mk_kernels_bf16_4w(int kind);
void* mk_kernels_bf16_8w(int kind);
void* mk_kernels_bf16_16w(int kind);
void* mk_kernels_f32_1(int kind);
void* mk_kernels_f32_2(int kind);
void* mk_kernels_f32_4(int kind);
}
