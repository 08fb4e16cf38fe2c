"""Plain CPU oracle for the QSA MQA indexer.  Test infrastructure only: the
product library never imports it."""
