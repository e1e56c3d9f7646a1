// Kernels for bf16 I/O with the elu1 feature map.
#define SLIM_IO_T __bf16
#define SLIM_FEAT FEAT_ELU1
#define SLIM_FEAT_IS_FAVOR 0
#define SLIM_TABLE_FN table_bf16_elu1
#include "slim_inst.inc"
