// dW-pass kernels for f32 I/O with the favor feature map.
#define SLIM_IO_T float
#define SLIM_FEAT FEAT_FAVOR
#define SLIM_FEAT_IS_FAVOR 1
#define SLIM_DW_TU 1
#define SLIM_TABLE_FN table_f32_favor_dw
#include "slim_inst.inc"
