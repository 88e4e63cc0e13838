// fa_main_softcap_dropout.hip -- the instantiations of the key-tile kernel of
// fa_main.hip with both soft-capped scores and dropout, in a translation unit
// of their own so that they compile in parallel with the rest.
#define FA_TU_SOFTCAP 1
#define FA_TU_DROPOUT 1
#include "fa_main.hip"
